// Weighted gather of the expert outputs back into token order.
//
// The Ling-2.6-1T page, §1 (scatter -> local expert FFN -> gather results)
// and §5 (the shared expert's output is added to the routed result); the
// sglang-jax gap list, §8 (gather-reduce: a weighted reduction of each
// token's top-k rows); the Kimi K3 page, §2.4 (routed_expert_norm: an RMSNorm
// of the routed sum before the up-projection, with the shared experts on a
// separate path).
//
// One workgroup per token (with RMSNorm, which needs the whole row), or per
// token and slice of 256 chunks (without: more workgroups for small T).
// Each thread owns CPT chunks of 8 channels, reads
// the k fp32 expert rows with 16-byte loads (coalesced along the row, a few
// pairs' loads in flight at once),
// accumulates w_j * y in fp32 in slot order, optionally normalises, adds the
// shared row and stores bf16 (round to nearest even): the output is rounded
// once.
#include <math.h>

#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace moe {

template <int CPT>
__global__ __launch_bounds__(1024) void combine_kernel(const float* __restrict__ y_rows,
                                                       const int* __restrict__ pair_to_row,
                                                       const float* __restrict__ topk_w, int H,
                                                       int k, const float* __restrict__ y_shared,
                                                       const float* __restrict__ gamma, float eps,
                                                       uint16_t* __restrict__ out) {
  __shared__ float red[16];
  const long t = blockIdx.x;
  const int nchk = H >> 3;
  float acc[CPT][8];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;

  // this workgroup's slice of the row's chunks (the whole row when gridDim.y = 1)
  const int base = blockIdx.y * blockDim.x * CPT;
  // the shared row's loads go out with the first pairs' (it is added last;
  // wide rows, CPT > 2, load it at the end to keep their registers)
  constexpr bool kEarlyShared = CPT <= 2;
  float4 sh[kEarlyShared ? CPT : 1][2];
  if (kEarlyShared && y_shared) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = base + threadIdx.x + c * blockDim.x;
      if (idx < nchk) {
        const float4* src = reinterpret_cast<const float4*>(y_shared + t * H);
        sh[c][0] = src[2 * idx];
        sh[c][1] = src[2 * idx + 1];
      }
    }
  }
  // pairs in batches of KB: a batch's rows and weights are read first, then
  // all of its row loads are issued, then summed in slot order (the same sum
  // as one pair at a time, without a round trip per pair)
  constexpr int KB = CPT == 1 ? 4 : (CPT == 2 ? 2 : 1);
  for (int j0 = 0; j0 < k; j0 += KB) {
    int r[KB];
    float w[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const bool in = j0 + j < k;
      r[j] = in ? pair_to_row[t * k + j0 + j] : -1;
      w[j] = in ? topk_w[t * k + j0 + j] : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = base + threadIdx.x + c * blockDim.x;
      if (idx >= nchk) continue;
      float4 v[KB][2];
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (r[j] >= 0) {
          const float4* src = reinterpret_cast<const float4*>(y_rows + (long)r[j] * H);
          v[j][0] = src[2 * idx];
          v[j][1] = src[2 * idx + 1];
        }
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (r[j] < 0) continue;
        const float4 v0 = v[j][0], v1 = v[j][1];
        const float wj = w[j];
        acc[c][0] += wj * v0.x; acc[c][1] += wj * v0.y; acc[c][2] += wj * v0.z; acc[c][3] += wj * v0.w;
        acc[c][4] += wj * v1.x; acc[c][5] += wj * v1.y; acc[c][6] += wj * v1.z; acc[c][7] += wj * v1.w;
      }
    }
  }

  if (gamma) {
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += acc[c][i] * acc[c][i];
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = base + threadIdx.x + c * blockDim.x;
      if (idx < nchk) {
        const float4 g0 = reinterpret_cast<const float4*>(gamma)[2 * idx];
        const float4 g1 = reinterpret_cast<const float4*>(gamma)[2 * idx + 1];
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[c][i] = acc[c][i] * inv * g[i];
      }
    }
  }

#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = base + threadIdx.x + c * blockDim.x;
    if (idx >= nchk) continue;
    if (y_shared) {
      float4 v0, v1;
      if constexpr (kEarlyShared) {
        v0 = sh[c][0];
        v1 = sh[c][1];
      } else {
        const float4* src = reinterpret_cast<const float4*>(y_shared + t * H);
        v0 = src[2 * idx];
        v1 = src[2 * idx + 1];
      }
      acc[c][0] += v0.x; acc[c][1] += v0.y; acc[c][2] += v0.z; acc[c][3] += v0.w;
      acc[c][4] += v1.x; acc[c][5] += v1.y; acc[c][6] += v1.z; acc[c][7] += v1.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = bf16_rne(acc[c][2 * q]) | (bf16_rne(acc[c][2 * q + 1]) << 16);
    reinterpret_cast<uint4*>(out + t * H)[idx] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_combine(const float* y_rows, const int* pair_to_row, const float* w, int T,
                          int H, int k, const float* y_shared, const float* gamma, float eps,
                          uint16_t* out, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (T == 0) return hipSuccess;
  const int chunks = H / 8;
  int cpt = 1, threads, slices = 1;
  if (gamma) {   // the norm needs the whole row in one workgroup
    while (chunks > 1024 * cpt) cpt *= 2;
    threads = (chunks + cpt - 1) / cpt;
    threads = ((threads + 63) / 64) * 64;
  } else {       // one chunk per thread, slices of 256 chunks
    threads = chunks < 256 ? ((chunks + 63) / 64) * 64 : 256;
    slices = (chunks + threads - 1) / threads;
  }
#define MOE_CB(C)                                                                                          \
  hipExtLaunchKernelGGL(combine_kernel<C>, dim3(T, slices), dim3(threads), 0, s, ev_start, ev_stop, 0, y_rows, \
                        pair_to_row, w, H, k, y_shared, gamma, eps, out)
  switch (cpt) {
    case 1: MOE_CB(1); break;
    case 2: MOE_CB(2); break;
    case 4: MOE_CB(4); break;
    default: MOE_CB(8); break;
  }
#undef MOE_CB
  return hipGetLastError();
}

}  // namespace moe
