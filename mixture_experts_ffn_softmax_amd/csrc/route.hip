// Softmax router with top-k selection: one wavefront per token.
//
// The k experts with the largest logits are chosen in k rounds of a
// wave-wide arg-max over the key (logit, -expert index), so equal logits go
// to the lower index and the slots come out in descending order.  The raw
// fp32 logits decide the selection, which therefore does not depend on the
// rounding of exp.  Weights: w_j = exp(l_j - l_max) / sum_sel exp(l - l_max),
// which equals p_j / sum_sel p for p = softmax over all experts; with the
// sigmoid score (the Kimi K3 page, §2.4) p_j = 1 / (1 + e^-l_j), which is
// increasing in the logit too, so the selection is the same.
// Top-8 of 256 routed experts on the Ling-2.6-1T page (overview, §1 cost
// model); renormalised top-k weights on the Kimi K3 page, §2.4.
#include <math.h>

#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace moe {

constexpr int kRouteSlots = kMaxExperts / 64;  // logits held per lane

__device__ __forceinline__ bool route_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// SLOTS: logits held per lane (E <= 64 * SLOTS), so that each round scans
// only the slots the expert count needs.
template <int SLOTS>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, bool sigmoid, int* __restrict__ ids,
                                                    float* __restrict__ w) {
  static_assert(SLOTS <= kRouteSlots, "at most kMaxExperts experts");
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  const int slots = (E + 63) >> 6;

  float v[SLOTS];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = i * 64 + lane;
    const bool ok = (i < slots) && (e < E);
    const float l = ok ? row[e] : 0.0f;
    v[i] = (l == l) ? l : -INFINITY;   // a NaN logit ranks below every number
    avail |= ok ? (1u << i) : 0u;
  }

  float vmax = 0.0f, sum = 0.0f, mine = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int e = i * 64 + lane;
      if (((avail >> i) & 1u) && route_better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (route_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) avail &= ~(1u << (bi >> 6));
    if (j == 0) vmax = bv;
    const float ex = sigmoid ? 1.0f / (1.0f + expf(-bv)) : expf(bv - vmax);
    sum += ex;
    if (lane == j) {
      my_id = bi;
      mine = ex;
    }
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = mine / sum;
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, bool sigmoid, int* ids, float* w,
                        hipStream_t s, hipEvent_t ev_start) {
  if (T == 0) return hipSuccess;
#define MOE_RT(S) \
  hipExtLaunchKernelGGL(route_kernel<S>, dim3((T + 3) / 4), dim3(256), 0, s, ev_start, nullptr, 0, logits, T, E, k, \
                        sigmoid, ids, w)
  if (E <= 64) MOE_RT(1);
  else if (E <= 256) MOE_RT(4);
  else MOE_RT(kRouteSlots);
#undef MOE_RT
  return hipGetLastError();
}

}  // namespace moe
