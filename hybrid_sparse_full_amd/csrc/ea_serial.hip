// Serial dispatch of a hybrid-head layer: the baseline that the Elastic
// Attention notes compare their fused kernel against (English notes, 04
// Deployment, Algorithm 1 (a) and Figure 4; Chinese notes, 05 Deployment).
// The heads are split by mode into a "full" group and a "sparse" group with
// explicit copies, each group runs as its own single-mode layer, and both
// outputs are written back into the layer's tensors.  Every copy here is a
// plain HBM-bound kernel: 16 bytes per thread, consecutive threads on
// consecutive bytes of one head row.
#include "ea_device.h"

namespace ea {

// dst[t, j, :] = src[t, map.idx[j], :] for j < map.n (bf16 rows of D).
template <int D>
__global__ __launch_bounds__(256) void k_gather_heads(const uint16_t* __restrict__ src, int32_t hs,
                                                      uint16_t* __restrict__ dst, HeadMap map,
                                                      int64_t T) {
  constexpr int CPR = D / 8;  // 16-byte chunks per head row
  const int64_t n = T * map.n * CPR;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i % CPR);
    const int64_t r = i / CPR;
    const int j = (int)(r % map.n);
    const int64_t t = r / map.n;
    *(uint4*)(dst + i * 8) = *(const uint4*)(src + ((t * hs + map.idx[j]) * D + c * 8));
  }
}

// dst[t, map.idx[j], :] = src[t, j, :] and lse_dst[map.idx[j], t] = lse_src[j, t].
template <int D>
__global__ __launch_bounds__(256) void k_scatter_heads(const uint16_t* __restrict__ src,
                                                       const float* __restrict__ lse_src,
                                                       uint16_t* __restrict__ dst, int32_t hd,
                                                       float* __restrict__ lse_dst, HeadMap map,
                                                       int64_t T) {
  constexpr int CPR = D / 8;
  const int64_t n = T * map.n * CPR;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i % CPR);
    const int64_t r = i / CPR;
    const int j = (int)(r % map.n);
    const int64_t t = r / map.n;
    *(uint4*)(dst + ((t * hd + map.idx[j]) * D + c * 8)) = *(const uint4*)(src + i * 8);
  }
  const int64_t nl = T * map.n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nl; i += (int64_t)gridDim.x * 256) {
    const int j = (int)(i / T);
    const int64_t t = i % T;
    lse_dst[(int64_t)map.idx[j] * T + t] = lse_src[i];
  }
}

__global__ __launch_bounds__(256) void k_fill_u8(uint8_t* __restrict__ p, int64_t n, uint8_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = v;
}

static unsigned copy_grid(int64_t work) {
  const int64_t b = (work + 255) / 256;
  return (unsigned)(b < 1 ? 1 : b > 65536 ? 65536 : b);
}

hipError_t launch_gather_heads(int D, const uint16_t* src, int32_t hs, uint16_t* dst,
                               const HeadMap& map, int64_t T, hipStream_t st) {
  if (map.n == 0 || T == 0) return hipSuccess;
  const unsigned g = copy_grid(T * map.n * (D / 8));
  if (D == 128) hipLaunchKernelGGL(k_gather_heads<128>, dim3(g), dim3(256), 0, st, src, hs, dst, map, T);
  else hipLaunchKernelGGL(k_gather_heads<64>, dim3(g), dim3(256), 0, st, src, hs, dst, map, T);
  return hipGetLastError();
}

hipError_t launch_scatter_heads(int D, const uint16_t* src, const float* lse_src, uint16_t* dst,
                                int32_t hd, float* lse_dst, const HeadMap& map, int64_t T,
                                hipStream_t st) {
  if (map.n == 0 || T == 0) return hipSuccess;
  const unsigned g = copy_grid(T * map.n * (D / 8));
  if (D == 128)
    hipLaunchKernelGGL(k_scatter_heads<128>, dim3(g), dim3(256), 0, st, src, lse_src, dst, hd, lse_dst, map, T);
  else
    hipLaunchKernelGGL(k_scatter_heads<64>, dim3(g), dim3(256), 0, st, src, lse_src, dst, hd, lse_dst, map, T);
  return hipGetLastError();
}

hipError_t launch_fill_u8(uint8_t* p, int64_t n, uint8_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u8, dim3(copy_grid(n)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace ea
