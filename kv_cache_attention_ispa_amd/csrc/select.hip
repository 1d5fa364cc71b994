// Layer selection (gfx950).
//
// After the warmup every layer has a reconstruction error epsilon (technical summary, gist.science
// nl/pt, section 2 "Dynamic layer selection"): the layers whose history the absorbed weights
// reproduce best are the ones converted to local attention.  This kernel ranks the per-layer errors
// where they were computed, on the device, and writes the role map the inference stage follows.
//
// Order: ascending epsilon; equal values keep the lower layer index first (a stable sort); NaN ranks
// after every number, and a layer whose factorisation failed (info != 0: its epsilon is undefined)
// ranks as NaN.  The first k in that order are converted, except those whose epsilon is NaN (their
// absorbed weights are undefined), so fewer than k are converted when fewer than k errors are
// numbers.  Layer i's rank is the number of
// layers that come before it in that order, so ranks are a permutation of 0 .. n - 1 and each thread
// finds its layer's rank by one pass over the errors held in LDS.
#include "../../include/ispa.h"
#include "common.hpp"

namespace ispa {
namespace {

constexpr int kMaxLayers = 4096;

__device__ __forceinline__ bool ranks_before(float a, int ia, float b, int ib) {
  const bool na = a != a, nb = b != b;
  if (na != nb) return nb;
  if (!na && a != b) return a < b;
  return ia < ib;
}

__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ eps,
                                                      const int32_t* __restrict__ info, int n, int k,
                                                      int32_t* __restrict__ role, int32_t* __restrict__ order) {
  __shared__ float e[kMaxLayers];
  for (int i = threadIdx.x; i < n; i += blockDim.x) e[i] = (info && info[i] != 0) ? __builtin_nanf("") : eps[i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float x = e[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += ranks_before(e[j], j, x, i) ? 1 : 0;
    role[i] = rank < k && x == x ? 1 : 0;
    if (order) order[rank] = i;
  }
}

}  // namespace
}  // namespace ispa

extern "C" int ispa_select_layers(int n_layers, const float* eps, const int32_t* info, int k, int32_t* role,
                                  int32_t* order, void* stream) {
  if (n_layers < 1 || n_layers > ispa::kMaxLayers || k < 0 || k > n_layers) return ISPA_EINVAL;
  if (!eps || !role) return ISPA_EINVAL;
  if (((uintptr_t)eps & 3) || ((uintptr_t)info & 3) || ((uintptr_t)role & 3) || ((uintptr_t)order & 3))
    return ISPA_EINVAL;
  hipLaunchKernelGGL(ispa::select_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, eps, info, n_layers, k, role,
                     order);
  return hipGetLastError() == hipSuccess ? ISPA_OK : ISPA_EHIP;
}
