// Attention Router, inference pass: boundary pooling of the key states, the
// Task MLP and the Router MLP, and the arg max that writes each (sequence,
// KV head)'s mode (English paper-reading notes, 03 Method, Figure 3 (b)(c);
// Chinese notes, 04 Method).
//
// One workgroup of 256 threads per (sequence, KV head).  The work is tiny
// (about 0.26 M multiply-adds per head at d = 128, H = 512) and entirely
// latency-bound, so everything stays in one workgroup and in LDS: the pooled
// vector and the Task MLP output (2 d floats), one hidden layer (H floats) and
// a reduction buffer.  Weight reads are coalesced: a thread owns one output
// column and walks the rows of a row-major [in][out] matrix, so the threads
// of a wave read consecutive addresses of one row at a time.  The pooling
// reads the 2 d bytes of one token and head with D consecutive threads.
// Sums run in fp32 in a fixed order, so the result is deterministic.
#include "ea_device.h"

namespace ea {

constexpr int ROUTER_NT = 256;
constexpr int ROUTER_HMAX = 1024;

struct RouterArgs {
  const uint16_t* k;
  const int32_t* cu;
  ea_router_desc w;
  int32_t nseq, Hkv, T, maxL;
  uint8_t retrieval_mode, sparse_mode;
  uint8_t* modes;
  float* logits;
};

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int D>
__global__ __launch_bounds__(ROUTER_NT) void k_route(RouterArgs a) {
  constexpr int NG = ROUTER_NT / D;  // thread groups over one D-vector
  __shared__ float xu[2 * D];        // pooled keys x, then the Task MLP output u
  __shared__ float hid[ROUTER_HMAX];
  __shared__ float red[ROUTER_NT];
  const int tid = threadIdx.x;
  const int grp = tid / D, c = tid % D;
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int H = a.w.hidden;

  // Sequence bounds, clamped into [0, T) with the length capped at maxL.
  const int32_t s0 = min(max(a.cu[b], 0), a.T);
  const int32_t e0 = min(min(max(a.cu[b + 1], s0), a.T), s0 + a.maxL);
  const int32_t L = e0 - s0;
  // Boundary set: local tokens [0, h0) and [t0, L), t0 >= h0, each once.
  const int32_t h0 = min(a.w.pool_head, L);
  const int32_t t0 = max(L - a.w.pool_tail, h0);
  const int32_t n = h0 + (L - t0);

  // 1. Mean pooling.  Group grp takes every NG-th pooled token.
  float part = 0.f;
  for (int32_t p = grp; p < n; p += NG) {
    const int32_t t = p < h0 ? p : t0 + (p - h0);
    part += bf16_bits_to_float(a.k[((size_t)(s0 + t) * a.Hkv + g) * D + c]);
  }
  red[tid] = part;
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) s += red[q * D + tid];
    xu[tid] = n > 0 ? s / (float)n : 0.f;
  }
  __syncthreads();

  // 2. Task MLP, hidden layer: hid = relu(x W1 + b1).
  for (int j = tid; j < H; j += ROUTER_NT) {
    float acc = a.w.b1[j];
    for (int i = 0; i < D; ++i) acc = fmaf(xu[i], a.w.w1[(size_t)i * H + j], acc);
    hid[j] = fmaxf(acc, 0.f);
  }
  __syncthreads();

  // 3. Task MLP output u = hid W2 + b2; group grp sums every NG-th hidden unit.
  part = 0.f;
  for (int j = grp; j < H; j += NG) part = fmaf(hid[j], a.w.w2[(size_t)j * D + c], part);
  red[tid] = part;
  __syncthreads();
  if (tid < D) {
    float s = a.w.b2[tid];
#pragma unroll
    for (int q = 0; q < NG; ++q) s += red[q * D + tid];
    xu[D + tid] = s;
  }
  __syncthreads();

  // 4. Router MLP, hidden layer: hid = relu([x, u] W3 + b3).
  for (int j = tid; j < H; j += ROUTER_NT) {
    float acc = a.w.b3[j];
    for (int i = 0; i < 2 * D; ++i) acc = fmaf(xu[i], a.w.w3[(size_t)i * H + j], acc);
    hid[j] = fmaxf(acc, 0.f);
  }
  __syncthreads();

  // 5. Logits z = hid W4 + b4, then the arg max (ties to the retrieval mode).
  float p0 = 0.f, p1 = 0.f;
  for (int j = tid; j < H; j += ROUTER_NT) {
    p0 = fmaf(hid[j], a.w.w4[2 * j], p0);
    p1 = fmaf(hid[j], a.w.w4[2 * j + 1], p1);
  }
  p0 = wave_sum(p0);
  p1 = wave_sum(p1);
  if ((tid & 63) == 0) {
    red[2 * (tid >> 6)] = p0;
    red[2 * (tid >> 6) + 1] = p1;
  }
  __syncthreads();
  if (tid == 0) {
    float z0 = a.w.b4[0], z1 = a.w.b4[1];
#pragma unroll
    for (int w = 0; w < ROUTER_NT / 64; ++w) {
      z0 += red[2 * w];
      z1 += red[2 * w + 1];
    }
    const size_t o = (size_t)b * a.Hkv + g;
    a.modes[o] = z1 > z0 ? a.sparse_mode : a.retrieval_mode;
    if (a.logits) {
      a.logits[2 * o] = z0;
      a.logits[2 * o + 1] = z1;
    }
  }
}

hipError_t launch_route(const EaDims& d, const ea_router_desc& w, const uint16_t* k,
                        const int32_t* cu, uint8_t retrieval_mode, uint8_t sparse_mode,
                        uint8_t* modes, float* logits, hipStream_t st) {
  RouterArgs a;
  a.k = k;
  a.cu = cu;
  a.w = w;
  a.nseq = d.nseq;
  a.Hkv = d.Hkv;
  a.T = d.T;
  a.maxL = d.maxL;
  a.retrieval_mode = retrieval_mode;
  a.sparse_mode = sparse_mode;
  a.modes = modes;
  a.logits = logits;
  const dim3 grid((unsigned)((int64_t)d.nseq * d.Hkv));
  if (d.D == 128) hipLaunchKernelGGL(k_route<128>, grid, dim3(ROUTER_NT), 0, st, a);
  else hipLaunchKernelGGL(k_route<64>, grid, dim3(ROUTER_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace ea
