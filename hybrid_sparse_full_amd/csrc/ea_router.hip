// Attention Router, inference pass: boundary pooling of the key states, the
// Task MLP and the Router MLP, and the arg max that writes each (sequence,
// KV head)'s mode (English paper-reading notes, 03 Method, Figure 3 (b)(c);
// Chinese notes, 04 Method).
//
// One workgroup of 1024 threads per (sequence, KV head).  The work is tiny
// (about 0.26 M multiply-adds per head at d = 128, H = 512) and bound by the
// latency of its dependent steps, so the design maximises loads in flight:
// every matrix-vector product splits its input dimension over thread groups
// (each thread issues all of its few float4 weight loads at once, four
// output columns per load, coalesced along the row-major [in][out] weights)
// and the partial sums meet in LDS.  The pooling spreads the boundary tokens
// over 1024 / d thread groups in the same way.  Sums run in fp32 in a fixed
// order, so the result is deterministic.
#include "ea_device.h"

namespace ea {

constexpr int ROUTER_NT = 1024;
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

// out[j] = act(bias[j] + sum_i in[i] W[i][j]) for j < nout (nout % 4 == 0),
// W row-major [nin][nout], 16-byte aligned rows.  Thread t takes the column
// quad jq = t % nq and the inputs i = ig, ig + IG, ... with ig = t / nq.
// part needs IG * nout <= 4 * ROUTER_NT floats.  Ends with a barrier.
template <bool RELU>
__device__ inline void matvec(const float* in, int nin, const float* __restrict__ W,
                              const float* __restrict__ bias, int nout, float* out, float* part) {
  const int tid = threadIdx.x;
  const int nq = nout / 4;
  const int IG = ROUTER_NT / nq;
  const int jq = tid % nq, ig = tid / nq;
  if (ig < IG) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = ig; i < nin; i += IG) {
      const f32x4 w = *(const f32x4*)(W + (size_t)i * nout + 4 * jq);
      const float x = in[i];
      acc[0] = fmaf(x, w[0], acc[0]);
      acc[1] = fmaf(x, w[1], acc[1]);
      acc[2] = fmaf(x, w[2], acc[2]);
      acc[3] = fmaf(x, w[3], acc[3]);
    }
    *(f32x4*)(part + ig * nout + 4 * jq) = acc;
  }
  __syncthreads();
  for (int j = tid; j < nout; j += ROUTER_NT) {
    float s = bias[j];
    for (int g = 0; g < IG; ++g) s += part[g * nout + j];
    out[j] = RELU ? fmaxf(s, 0.f) : s;
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(ROUTER_NT) void k_route(RouterArgs a) {
  constexpr int NG = ROUTER_NT / D;  // thread groups over one D-vector
  __shared__ float xu[2 * D];        // pooled keys x, then the Task MLP output u
  __shared__ float hid[ROUTER_HMAX];
  __shared__ __attribute__((aligned(16))) float part[4 * ROUTER_NT];
  const int tid = threadIdx.x;
  const int grp = tid / D, c = tid % D;
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int H = a.w.hidden;

  // Sequence bounds, clamped into [0, T) with the length capped at maxL.
  const int32_t s0 = min(max(a.cu[b], 0), a.T);
  const int32_t e0 = (int32_t)min<int64_t>(min(max(a.cu[b + 1], s0), a.T), (int64_t)s0 + a.maxL);
  const int32_t L = e0 - s0;
  // Boundary set: local tokens [0, h0) and [t0, L), t0 >= h0, each once.
  const int32_t h0 = min(a.w.pool_head, L);
  const int32_t t0 = max(L - a.w.pool_tail, h0);
  const int32_t n = h0 + (L - t0);

  // 1. Mean pooling.  Group grp takes every NG-th pooled token.
  float acc = 0.f;
  for (int32_t p = grp; p < n; p += NG) {
    const int32_t t = p < h0 ? p : t0 + (p - h0);
    acc += bf16_bits_to_float(a.k[((size_t)(s0 + t) * a.Hkv + g) * D + c]);
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) s += part[q * D + tid];
    xu[tid] = n > 0 ? s / (float)n : 0.f;
  }
  __syncthreads();

  // 2. Task MLP: hid = relu(x W1 + b1), u = hid W2 + b2.
  matvec<true>(xu, D, a.w.w1, a.w.b1, H, hid, part);
  matvec<false>(hid, H, a.w.w2, a.w.b2, D, xu + D, part);
  // 3. Router MLP, hidden layer: hid = relu([x, u] W3 + b3).
  matvec<true>(xu, 2 * D, a.w.w3, a.w.b3, H, hid, part);

  // 4. Logits z = hid W4 + b4, then the arg max (ties to the retrieval mode).
  float p0 = 0.f, p1 = 0.f;
  for (int j = tid; j < H; j += ROUTER_NT) {
    p0 = fmaf(hid[j], a.w.w4[2 * j], p0);
    p1 = fmaf(hid[j], a.w.w4[2 * j + 1], p1);
  }
  p0 = wave_sum(p0);
  p1 = wave_sum(p1);
  if ((tid & 63) == 0) {
    part[2 * (tid >> 6)] = p0;
    part[2 * (tid >> 6) + 1] = p1;
  }
  __syncthreads();
  if (tid == 0) {
    float z0 = a.w.b4[0], z1 = a.w.b4[1];
#pragma unroll
    for (int w = 0; w < ROUTER_NT / 64; ++w) {
      z0 += part[2 * w];
      z1 += part[2 * w + 1];
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
