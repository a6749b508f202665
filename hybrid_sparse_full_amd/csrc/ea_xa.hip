// XA block selection: antidiagonal scoring (k_xa_score) and the integer
// top-mass selector (k_xa_select).
//
// Scoring is a causal bf16 GEMM over "reduced" rows: reduced query a is the
// concatenation of the S query rows aS..aS+S-1 (length S*d) and reduced key
// b' the concatenation of key rows b'S+S-1..b'S (reversed), so their dot
// product is the sum of the stride-S antidiagonal entries of that S x S
// sub-tile of Q K^T.  The MFMA tile computes S~^T = K~ Q~^T, which puts one
// reduced query per lane and the reduced keys of a block in registers; the
// epilogue turns every (reduced row a, block J) pair into one log-sum-exp
//     lse2[a, J] = log2 sum_{b' in J, b' <= a} exp2(c * log2(e) * s^[a, b']),
// so the row softmax never needs a second pass over the GEMM: the selector
// normalises per row from these partial sums.
#include "ea_device.h"

namespace ea {

constexpr int XT = 128;  // reduced rows / columns per tile
constexpr int XK = 64;   // k-chunk (bf16 elements) staged in LDS

__device__ inline int64_t tri_root(int64_t loc) {
  int64_t t = (int64_t)((sqrt(8.0 * (double)loc + 1.0) - 1.0) * 0.5);
  while (tri64(t + 1) <= loc) ++t;
  while (tri64(t) > loc) --t;
  return t;
}

template <int D, int R>
__global__ __launch_bounds__(256) void k_xa_score(EaDims d, const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k, SeqMeta m,
                                                  const int32_t* __restrict__ pair_bh,
                                                  const int64_t* __restrict__ pair_items,
                                                  float* __restrict__ lse_ws) {
  __shared__ __attribute__((aligned(16))) uint16_t As[XT * XK];  // K~ rows (b')
  __shared__ __attribute__((aligned(16))) uint16_t Bs[XT * XK];  // Q~ rows (a)
  __shared__ int64_t item_s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int wy = wave >> 1, wx = wave & 1;
  const int npairs = m.scal[SCAL_XA_PAIRS];
  const int64_t total = pair_items[npairs];
  unsigned long long* ctr = (unsigned long long*)(m.scal + SCAL_CTR64);
  const float C2 = d.scale * LOG2E;
  const int S = d.S;

  while (true) {
    if (tid == 0) item_s = (int64_t)atomicAdd(ctr, 1ull);
    __syncthreads();
    const int64_t item = item_s;
    __syncthreads();
    if (item >= total) break;
    const int p = upper_index(pair_items, npairs + 1, item);
    const int64_t loc = item - pair_items[p];
    const int64_t ta = tri_root(loc);
    const int64_t tb = loc - tri64(ta);
    const int32_t bh = pair_bh[p];
    const int b = bh / d.Hq, h = bh % d.Hq, g = h / d.G;
    const int64_t tok0 = m.start[b];
    const int32_t len = m.len[b];
    const int32_t nred = len / S;
    const int64_t nqb = len / d.B;
    const int32_t a0 = (int32_t)ta * XT, b0 = (int32_t)tb * XT;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int k0 = 0; k0 < S * D; k0 += XK) {
      const int t = k0 / D, dk = k0 % D;
#pragma unroll
      for (int c = tid; c < XT * 8; c += 256) {
        const int row = c >> 3, ch = c & 7;
        const int sw = ((ch ^ (row & 7)) * 8);
        uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
        const int32_t bq = b0 + row, aq = a0 + row;
        if (bq < nred)
          kv = *(const uint4*)(k + ((tok0 + (int64_t)bq * S + (S - 1 - t)) * d.Hkv + g) * D + dk + ch * 8);
        if (aq < nred)
          qv = *(const uint4*)(q + ((tok0 + (int64_t)aq * S + t) * d.Hq + h) * D + dk + ch * 8);
        *(uint4*)(As + row * XK + sw) = kv;
        *(uint4*)(Bs + row * XK + sw) = qv;
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < XK / 16; ++ks) {
        const int chunk = 2 * ks + half;
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = wy * 64 + 32 * i + l32;
          af[i] = *(const bf16x8*)(As + row * XK + ((chunk ^ (row & 7)) * 8));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = wx * 64 + 32 * j + l32;
          bfr[j] = *(const bf16x8*)(Bs + row * XK + ((chunk ^ (row & 7)) * 8));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }

    // Epilogue: per (reduced row a, block J) log-sum-exp in log2 units.
    const int64_t base_bh = (int64_t)R * (m.tri_prefix[b] * d.Hq + (int64_t)h * tri64(nqb));
    constexpr int NG = 32 / R;      // block groups per 32-row MFMA tile
    constexpr int RPG = R / 2;      // registers per group per lane
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int32_t a = a0 + wx * 64 + 32 * j + l32;
        const int32_t Ia = a / R;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const int32_t brow0 = b0 + wy * 64 + 32 * i + gi * R;
          const int32_t J = brow0 / R;
          float v[RPG];
          float mloc = -INFINITY;
#pragma unroll
          for (int e = 0; e < RPG; ++e) {
            const int r = gi * RPG + e;
            const int32_t bq = b0 + wy * 64 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool ok = (bq <= a) && (a < nred);
            v[e] = ok ? acc[i][j][r] : -INFINITY;
            mloc = fmaxf(mloc, v[e]);
          }
          const float mm = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
          float s = 0.f;
          if (mm != -INFINITY) {
#pragma unroll
            for (int e = 0; e < RPG; ++e) s += exp2f((v[e] - mm) * C2);
          }
          s += __shfl_xor(s, 32, 64);
          if (half == 0 && a < nred && J <= Ia) {
            const int64_t idx = base_bh + (int64_t)R * tri64(Ia) + (int64_t)(a - R * Ia) * (Ia + 1) + J;
            lse_ws[idx] = mm * C2 + log2f(s);
          }
        }
      }
  }
}

// ---------------------------------------------------------------- selector
constexpr int SEL_NT = 256;

template <typename T>
__device__ inline T block_max_u(T v, T* smem) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) smem[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    T x = smem[0];
    for (int i = 1; i < SEL_NT / 64; ++i) x = smem[i] > x ? smem[i] : x;
    smem[SEL_NT / 64] = x;
  }
  __syncthreads();
  T res = smem[SEL_NT / 64];
  __syncthreads();
  return res;
}

template <int R>
__global__ __launch_bounds__(SEL_NT) void k_xa_select(EaDims d, const uint8_t* __restrict__ modes,
                                                      SeqMeta m, const float* __restrict__ lse_ws,
                                                      uint32_t* __restrict__ mask,
                                                      int32_t* __restrict__ row_count,
                                                      int64_t* __restrict__ xa_pairs,
                                                      float* __restrict__ block_mass) {
  extern __shared__ uint32_t dyn[];
  __shared__ float Mrow[R], Zrow[R];
  __shared__ uint64_t red[SEL_NT / 64 + 1];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int32_t qbg = (int32_t)(row / d.Hq);
  const int h = (int)(row % d.Hq);
  if (qbg >= m.scal[SCAL_TOTAL_QB]) return;
  const int32_t b = m.qb2seq[qbg];
  const int32_t I = qbg - m.qb_prefix[b];
  const int32_t len = m.len[b];
  const int mode = sane_mode(modes[(int64_t)b * d.Hkv + h / d.G]);
  uint32_t* mrow = mask + row * d.words;
  const int32_t nI = I + 1;
  if (mode != EA_MODE_XA) {
    for (int w = tid; w < d.words; w += SEL_NT) mrow[w] = 0u;
    if (tid == 0) row_count[row] = 0;
    return;
  }
  const int64_t B = d.B;
  if (len % d.B != 0) {
    // XA on a sequence that is not a whole number of blocks: every causal block.
    for (int w = tid; w < d.words; w += SEL_NT) {
      const int hi = I - w * 32;
      mrow[w] = hi < 0 ? 0u : (hi >= 31 ? 0xffffffffu : ((2u << hi) - 1u));
    }
    if (tid == 0) {
      row_count[row] = nI;
      const int64_t iend = min<int64_t>((int64_t)nI * B, len);
      atomicAdd((unsigned long long*)&xa_pairs[(int64_t)b * d.Hq + h],
                (unsigned long long)(tri64(iend) - tri64((int64_t)I * B)));
    }
    return;
  }

  const int64_t nqb = len / d.B;
  const float* base =
      lse_ws + (int64_t)R * (m.tri_prefix[b] * d.Hq + (int64_t)h * tri64(nqb)) + (int64_t)R * tri64(I);
  // 1. Per reduced row a: M_a = max_J lse2, Z_a = sum_J exp2(lse2 - M_a).
  {
    constexpr int TPR = SEL_NT / R;
    const int ar = tid / TPR, tj = tid % TPR;
    const float* rw = base + (int64_t)ar * nI;
    float mx = -INFINITY;
    for (int J = tj; J < nI; J += TPR) mx = fmaxf(mx, rw[J]);
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float z = 0.f;
    for (int J = tj; J < nI; J += TPR) z += exp2f(rw[J] - mx);
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
    if (tj == 0) {
      Mrow[ar] = mx;
      Zrow[ar] = z;
    }
  }
  __syncthreads();
  // 2. Block masses and integer weights.
  float* Pf = (float*)dyn;
  uint32_t* wv = dyn + d.maxqb;
  uint32_t* bits = dyn + 2 * d.maxqb;
  uint64_t wsum = 0;
  uint32_t wmax = 0;
  for (int J = tid; J < nI; J += SEL_NT) {
    float acc = 0.f;
#pragma unroll
    for (int ar = 0; ar < R; ++ar) acc += exp2f(base[(int64_t)ar * nI + J] - Mrow[ar]) / Zrow[ar];
    const float P = acc * (1.0f / R);
    Pf[J] = P;
    const float x = P * 16777216.0f;
    const float fl = floorf(x);
    uint32_t w = (uint32_t)fl + ((x - fl) >= 0.5f ? 1u : 0u);
    w = w < 1u ? 1u : w;
    wv[J] = w;
    wsum += w;
    wmax = w > wmax ? w : wmax;
  }
  for (int w = tid; w < d.words; w += SEL_NT) bits[w] = 0u;
  const uint64_t W = block_sum<SEL_NT, uint64_t>(wsum, red);
  const uint32_t Wmax = (uint32_t)block_max_u<uint64_t>((uint64_t)wmax, red);
  const uint64_t tn = (uint64_t)d.tau_num, td = (uint64_t)d.tau_den;
  const uint64_t target = tn * W;
  // 3. v* = largest v with (sum of w_J >= v) * td >= tn * W.
  uint32_t lo = 1, hi = Wmax + 1;
  while (hi - lo > 1) {
    const uint32_t mid = lo + (hi - lo) / 2;
    uint64_t s = 0;
    for (int J = tid; J < nI; J += SEL_NT) s += wv[J] >= mid ? wv[J] : 0u;
    const uint64_t F = block_sum<SEL_NT, uint64_t>(s, red);
    if (F * td >= target) lo = mid;
    else hi = mid;
  }
  const uint32_t vstar = lo;
  uint64_t sg = 0;
  for (int J = tid; J < nI; J += SEL_NT) sg += wv[J] > vstar ? wv[J] : 0u;
  const uint64_t Fgt = block_sum<SEL_NT, uint64_t>(sg, red);
  const uint64_t need = target - Fgt * td;  // > 0 by maximality of v*
  const uint64_t vt = (uint64_t)vstar * td;
  const uint64_t ceq = (need + vt - 1) / vt;  // blocks of weight v* to take, lowest J first
  // 4. Rank of each weight-v* block among equals (J order), then set bits.
  const int chunk = (nI + SEL_NT - 1) / SEL_NT;
  const int j0 = min(nI, tid * chunk), j1 = min(nI, j0 + chunk);
  uint64_t neq = 0;
  for (int J = j0; J < j1; ++J) neq += wv[J] == vstar;
  uint64_t tot_eq;
  uint64_t rank = block_exclusive_sum<SEL_NT, uint64_t>(neq, red, &tot_eq);
  for (int J = j0; J < j1; ++J) {
    bool sel = wv[J] > vstar || J == 0 || J == I;
    if (wv[J] == vstar) {
      sel = sel || rank < ceq;
      ++rank;
    }
    if (sel) atomicOr(&bits[J >> 5], 1u << (J & 31));
  }
  __syncthreads();
  uint64_t cnt = 0;
  for (int w = tid; w < d.words; w += SEL_NT) {
    mrow[w] = bits[w];
    cnt += __popc(bits[w]);
  }
  const uint64_t count = block_sum<SEL_NT, uint64_t>(cnt, red);
  if (tid == 0) {
    row_count[row] = (int32_t)count;
    const uint64_t pairs = (count - 1) * (uint64_t)(B * B) + (uint64_t)(B * (B + 1) / 2);
    atomicAdd((unsigned long long*)&xa_pairs[(int64_t)b * d.Hq + h], (unsigned long long)pairs);
  }
  if (block_mass) {
    float* bm = block_mass + row * d.maxqb;
    for (int J = tid; J < d.maxqb; J += SEL_NT) bm[J] = J < nI ? Pf[J] : 0.f;
  }
}

static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

hipError_t launch_xa_score(const EaDims& d, const uint16_t* q, const uint16_t* k, const SeqMeta& m,
                           void* ws, const WsLayout& L, hipStream_t st) {
  char* w = (char*)ws;
  const int32_t* pair_bh = (const int32_t*)(w + L.xa_pair_bh);
  const int64_t* pair_items = (const int64_t*)(w + L.xa_pair_items);
  float* lse = (float*)(w + L.xa_lse);
  const dim3 grid((unsigned)(device_cus() * 2));
#define EA_SCORE(DD, RR)                                                                      \
  hipLaunchKernelGGL((k_xa_score<DD, RR>), grid, dim3(256), 0, st, d, q, k, m, pair_bh, pair_items, lse)
  if (d.D == 128) {
    if (d.r == 8) EA_SCORE(128, 8);
    else if (d.r == 16) EA_SCORE(128, 16);
    else EA_SCORE(128, 32);
  } else {
    if (d.r == 8) EA_SCORE(64, 8);
    else if (d.r == 16) EA_SCORE(64, 16);
    else EA_SCORE(64, 32);
  }
#undef EA_SCORE
  return hipGetLastError();
}

hipError_t launch_xa_select(const EaDims& d, const uint8_t* modes, const SeqMeta& m, void* ws,
                            const WsLayout& L, uint32_t* mask, int32_t* row_count, int64_t* xa_pairs,
                            float* block_mass, hipStream_t st) {
  const float* lse = (const float*)((char*)ws + L.xa_lse);
  const size_t shm = (size_t)(2 * d.maxqb + d.words) * 4;
  const dim3 grid((unsigned)(d.nqb_max * d.Hq));
  if (d.r == 8)
    hipLaunchKernelGGL((k_xa_select<8>), grid, dim3(SEL_NT), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  else if (d.r == 16)
    hipLaunchKernelGGL((k_xa_select<16>), grid, dim3(SEL_NT), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  else
    hipLaunchKernelGGL((k_xa_select<32>), grid, dim3(SEL_NT), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  return hipGetLastError();
}

}  // namespace ea
