// Cross-partition combine of split-context decode: the partial results of
// each partition (running max m_p in log2 units, sum l_p, unnormalised o_p)
// are merged with the log-sum-exp identity into the final output.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "launch.h"
#include "pa_decode_common.h"

namespace pkv_decode {
namespace {

// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
// One workgroup of D threads per (query head, request), one output column per
// thread; only requests with more than one partition do work.  The (m_p, l_p)
// pairs are the same for every thread (broadcast loads) and all loads of a
// group of 16 partitions are issued before any is used, so a request's
// partials arrive in a few memory round trips instead of one per partition:
// with at most 32 partitions, one round trip for (m_p, l_p) and o_p together.
// Up to N partials in one round trip: every (m_p, l_p) and o_p loaded together,
// then combined.  (N fixed at compile time: 16 and 32 each fit their cases best.)
template <int N, int D>
__device__ __forceinline__ float combine_one_pass(const float2* ml, const float* o, int nparts) {
  float2 mlv[N];
  float ov[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const bool in = u < nparts;
    mlv[u] = in ? ml[u] : make_float2(-FLT_MAX, 0.f);
    ov[u] = in ? o[static_cast<int64_t>(u) * D] : 0.f;
  }
  float mmax = -FLT_MAX;
#pragma unroll
  for (int u = 0; u < N; ++u) mmax = fmaxf(mmax, mlv[u].x);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const float w = fast_exp2(mlv[u].x - mmax);
    den = fmaf(w, mlv[u].y, den);
    num = fmaf(w, ov[u], num);
  }
  return num / den;
}

template <int D>
__global__ __launch_bounds__(D) void pa_decode_reduce_kernel(DecodeParams p) {
  constexpr int U = 16;                      // partials per round trip, two-pass path
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int d = threadIdx.x;
  const int len = clamped_len(p, seq);
  // Partitions, plus the spare slot of a request whose shared prefix ends
  // inside a partition and that has tokens past it (slots 0..nparts-1 stay
  // contiguous).
  const int nparts =
      partials_of((len + p.part_tokens - 1) / p.part_tokens, shared_len(p, seq), len);
  if (nparts <= 1) return;
  const int64_t base = (static_cast<int64_t>(seq) * p.num_q_heads + h) * p.max_parts;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + base;
  const float* o = p.ws_o + base * D + d;
  float* const dst = p.out + (static_cast<int64_t>(seq) * p.num_q_heads + h) * D + d;
  if (nparts <= 16) {
    *dst = combine_one_pass<16, D>(ml, o, nparts);
    return;
  }
  if (nparts <= 32) {
    *dst = combine_one_pass<32, D>(ml, o, nparts);
    return;
  }
  float mmax = -FLT_MAX;
  for (int c = 0; c < nparts; c += U) {
    float mv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) mv[u] = c + u < nparts ? ml[c + u].x : -FLT_MAX;
#pragma unroll
    for (int u = 0; u < U; ++u) mmax = fmaxf(mmax, mv[u]);
  }
  float num = 0.f, den = 0.f;
  for (int c = 0; c < nparts; c += U) {
    float2 mlv[U];
    float ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = c + u < nparts;
      mlv[u] = in ? ml[c + u] : make_float2(-FLT_MAX, 0.f);
      ov[u] = in ? o[static_cast<int64_t>(c + u) * D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = fast_exp2(mlv[u].x - mmax);
      den = fmaf(w, mlv[u].y, den);
      num = fmaf(w, ov[u], num);
    }
  }
  *dst = num / den;
}

}  // namespace

hipError_t launch_reduce(const DecodeParams& prm, int head_dim, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(prm.num_q_heads), static_cast<unsigned>(prm.num_seqs));
  if (head_dim == 64)
    pkv::launch_kernel(pa_decode_reduce_kernel<64>, grid, dim3(64), 0, stream, prm);
  else
    pkv::launch_kernel(pa_decode_reduce_kernel<128>, grid, dim3(128), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace pkv_decode
