// One decode step of hybrid-head attention: the newest token of every
// sequence attends the cached keys that its KV head's mode keeps (routing
// from prefill is reused for every generated token: English paper-reading
// notes, 08 Commentary, the authors' stated limits; SSA = attention sink plus
// sliding window, glossary).  An XA head attends every cached key here:
// block selection needs blocks of query rows, and a decode step has one.
//
// A decode step reads each kept K/V row once and does 4 d flops per key and
// q-head, ~4 flop per byte: it is bound by HBM bandwidth, so it runs on the
// vector ALU with bf16 dot products, not on the matrix core.  Design:
//   * split-K: workgroup (split s, KV head g, sequence b) takes key-set
//     positions [1024 s, 1024 s + 1024) of its head's kept keys (the key set
//     is compressed: an SSA head's split 0 covers the sink and the start of
//     the window), for all G q-heads of g, so each K/V row is read once;
//   * 64 keys per step, one per lane: K rows and V rows of the next step are
//     loaded into registers while the current one is computed, then stored
//     to one of two LDS buffers.  K pieces (16 B) are XOR-swizzled within a
//     row so that the per-lane row reads are free of bank conflicts; V rows
//     are stored with consecutive key pairs interleaved per column, so that
//     P V is one v_dot2_f32_bf16 per key pair and column;
//   * scores: lane r computes c <q, k_r> with v_dot2_f32_bf16 (q read from
//     LDS as a broadcast); exact online softmax per step in the exp2 domain;
//     P is rounded to bf16 for the P V dot products (as in the prefill
//     kernel) while the row sum stays in fp32;
//   * each split writes (m, l, unnormalised o) in fp32; a second kernel
//     combines the splits of every (sequence, q-head) and writes o (bf16) and
//     lse (fp32).
#include "ea_device.h"

namespace ea {

constexpr int DEC_NT = 256;       // 4 waves
constexpr int DEC_KEYS = 64;      // keys per step (one per lane)

struct DecArgs {
  const uint16_t* q;   // [nseq, Hq, D]
  const uint16_t* k;   // [T, Hkv, D]
  const uint16_t* v;
  const int32_t* cu;
  const uint8_t* modes;
  float* part;         // [nseq, Hq, nsplit_max, D + 2]
  int32_t nseq, Hq, Hkv, G, T, maxL, sink, window, nsplit_max;
  float c2;            // softmax scale * log2(e)
};

// Kept keys of the decoded query (index L - 1) of a sequence of cached length L.
__device__ inline int32_t dec_kept(int mode, int32_t L, int32_t sink, int32_t window) {
  if (L <= 0) return 0;
  if (mode != EA_MODE_SSA) return L;
  const int32_t head = min(sink, L);
  return head + max(0, L - max(head, L - window));
}

// Key index of key-set position p (0 <= p < dec_kept).
__device__ inline int32_t dec_key(int mode, int32_t p, int32_t L, int32_t sink, int32_t window) {
  if (mode != EA_MODE_SSA) return p;
  const int32_t head = min(sink, L);
  return p < head ? p : max(head, L - window) + (p - head);
}

__device__ inline void seq_bounds(const DecArgs& a, int b, int32_t* s0, int32_t* L) {
  const int32_t s = min(max(a.cu[b], 0), a.T);
  const int32_t e = min(min(max(a.cu[b + 1], s), a.T), s + a.maxL);
  *s0 = s;
  *L = e - s;
}

template <int D, int HPW>
__global__ __launch_bounds__(DEC_NT) void k_decode(DecArgs a) {
  constexpr int NP = D / 8;                     // 16-byte pieces per row
  constexpr int KPIECES = DEC_KEYS * NP;        // K pieces per step
  constexpr int VUNITS = (DEC_KEYS / 2) * NP;   // V (key pair, piece) units per step
  constexpr int KPT = KPIECES / DEC_NT;         // per thread
  constexpr int VPT = VUNITS / DEC_NT;
  constexpr int CPL = D / 64;                   // output columns per lane
  static_assert(KPT >= 1 && VPT >= 1, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][DEC_KEYS * D];
  __shared__ __attribute__((aligned(16))) uint32_t vs[2][(DEC_KEYS / 2) * D];
  __shared__ __attribute__((aligned(16))) uint16_t qs[16 * D];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[4][DEC_KEYS];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  int mode = sane_mode(a.modes[(size_t)b * a.Hkv + g]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  const int32_t p0 = s * DEC_SPLIT;
  if (p0 >= n) return;  // uniform over the workgroup
  const int32_t p1 = min(n, p0 + DEC_SPLIT);
  const int nsteps = (p1 - p0 + DEC_KEYS - 1) / DEC_KEYS;

  // q of the group's G heads into LDS (bf16).
  for (int i = tid; i < a.G * NP; i += DEC_NT) {
    const int hh = i / NP, c = i % NP;
    *(uint4*)(qs + hh * D + c * 8) =
        *(const uint4*)(a.q + ((size_t)b * a.Hq + g * a.G + hh) * D + c * 8);
  }

  // Global -> registers for step t.
  uint4 kr[KPT], vr[VPT][2];
  auto load_step = [&](int t) {
    const int32_t base = p0 + t * DEC_KEYS;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * DEC_NT;
      const int r = idx / NP, c = idx % NP;
      const int32_t p = min(base + r, p1 - 1);
      const int32_t j = dec_key(mode, p, L, a.sink, a.window);
      kr[i] = *(const uint4*)(a.k + ((size_t)(s0 + j) * a.Hkv + g) * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * DEC_NT;
      const int rp = idx / NP, c = idx % NP;
      const int32_t pa = min(base + 2 * rp, p1 - 1), pb = min(base + 2 * rp + 1, p1 - 1);
      const int32_t ja = dec_key(mode, pa, L, a.sink, a.window);
      const int32_t jb = dec_key(mode, pb, L, a.sink, a.window);
      vr[i][0] = *(const uint4*)(a.v + ((size_t)(s0 + ja) * a.Hkv + g) * D + c * 8);
      vr[i][1] = *(const uint4*)(a.v + ((size_t)(s0 + jb) * a.Hkv + g) * D + c * 8);
    }
  };
  // Registers -> LDS buffer `buf`: K piece c of row r at physical piece
  // c ^ (r mod NP); V as key pairs interleaved per column: word (rp, col)
  // holds (v[2 rp][col], v[2 rp + 1][col]).
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * DEC_NT;
      const int r = idx / NP, c = idx % NP;
      *(uint4*)(ks[buf] + r * D + ((c ^ (r & (NP - 1))) * 8)) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * DEC_NT;
      const int rp = idx / NP, c = idx % NP;
      const uint32_t* x = (const uint32_t*)&vr[i][0];
      const uint32_t* y = (const uint32_t*)&vr[i][1];
      uint4 w0, w1;
      // low half of each word = key 2 rp, high half = key 2 rp + 1
      w0.x = __builtin_amdgcn_perm(y[0], x[0], 0x05040100u);
      w0.y = __builtin_amdgcn_perm(y[0], x[0], 0x07060302u);
      w0.z = __builtin_amdgcn_perm(y[1], x[1], 0x05040100u);
      w0.w = __builtin_amdgcn_perm(y[1], x[1], 0x07060302u);
      w1.x = __builtin_amdgcn_perm(y[2], x[2], 0x05040100u);
      w1.y = __builtin_amdgcn_perm(y[2], x[2], 0x07060302u);
      w1.z = __builtin_amdgcn_perm(y[3], x[3], 0x05040100u);
      w1.w = __builtin_amdgcn_perm(y[3], x[3], 0x07060302u);
      uint32_t* dst = vs[buf] + rp * D + c * 8;
      *(uint4*)dst = w0;
      *(uint4*)(dst + 4) = w1;
    }
  };

  // Per-head state: this wave owns heads wv, wv + 4, ... < G (HPW of them).
  float m[HPW], l[HPW], o[HPW][CPL];
#pragma unroll
  for (int u = 0; u < HPW; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[u][c] = 0.f;
  }

  load_step(0);
  for (int t = 0; t < nsteps; ++t) {
    const int buf = t & 1;
    store_step(buf);
    __syncthreads();
    if (t + 1 < nsteps) load_step(t + 1);
    const bool valid = p0 + t * DEC_KEYS + lane < p1;
    const uint16_t* krow = ks[buf] + lane * D;
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int hh = wv + 4 * u;
      if (hh >= a.G) break;  // wave-uniform
      // Score of key `lane`.
      float acc = 0.f;
      const uint16_t* qh = qs + hh * D;
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        const uint4 kk = *(const uint4*)(krow + ((c ^ (lane & (NP - 1))) * 8));
        const uint4 qq = *(const uint4*)(qh + c * 8);
        const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w}, qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]),
                                               __builtin_bit_cast(bf16x2, qw[e]), acc, false);
      }
      const float x = valid ? acc * a.c2 : -INFINITY;
      const float mn = fmaxf(m[u], wave_max(x));
      const float alpha = __builtin_amdgcn_exp2f(m[u] - mn);  // m = -inf at the start: 0
      const float p = __builtin_amdgcn_exp2f(x - mn);
      l[u] = l[u] * alpha + wave_sum(p);
      m[u] = mn;
      // P in bf16 pairs through LDS (this wave's own slice).
      pbuf[wv][lane] = __builtin_bit_cast(uint16_t, (__bf16)p);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint32_t* pp = (const uint32_t*)pbuf[wv];
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[u][c] *= alpha;
#pragma unroll
      for (int rp4 = 0; rp4 < DEC_KEYS / 2; rp4 += 4) {
        const uint4 p4 = *(const uint4*)(pp + rp4);
        const uint32_t pw[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t* vrow = vs[buf] + (rp4 + e) * D + CPL * lane;
          const bf16x2 pv = __builtin_bit_cast(bf16x2, pw[e]);
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            o[u][c] = __builtin_amdgcn_fdot2_f32_bf16(pv, __builtin_bit_cast(bf16x2, vrow[c]), o[u][c], false);
        }
      }
      // The next head's P overwrites pbuf after these reads.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }

  // Partial results of this split.
#pragma unroll
  for (int u = 0; u < HPW; ++u) {
    const int hh = wv + 4 * u;
    if (hh >= a.G) break;
    float* dst = a.part + (((size_t)b * a.Hq + g * a.G + hh) * a.nsplit_max + s) * (D + 2);
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[CPL * lane + c] = o[u][c];
    if (lane == 0) {
      dst[D] = m[u];
      dst[D + 1] = l[u];
    }
  }
}

// Combine the splits of one (sequence, q-head): 64 threads, CPL columns each.
template <int D>
__global__ __launch_bounds__(64) void k_decode_combine(DecArgs a, uint16_t* out, float* lse) {
  constexpr int CPL = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  int mode = sane_mode(a.modes[(size_t)b * a.Hkv + h / a.G]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  const int ns = (n + DEC_SPLIT - 1) / DEC_SPLIT;
  const float* src = a.part + ((size_t)b * a.Hq + h) * a.nsplit_max * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, src[s * (D + 2) + D]);
  float Ls = 0.f, acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(src[s * (D + 2) + D] - M);
    Ls += w * src[s * (D + 2) + D + 1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] += w * src[s * (D + 2) + CPL * lane + c];
  }
  uint16_t* orow = out + ((size_t)b * a.Hq + h) * D;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const float val = ns > 0 ? acc[c] / Ls : 0.f;
    orow[CPL * lane + c] = __builtin_bit_cast(uint16_t, (__bf16)val);
  }
  if (lane == 0) lse[(size_t)b * a.Hq + h] = ns > 0 ? (M + __log2f(Ls)) * LN2 : -INFINITY;
}

hipError_t launch_decode(const EaDims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* cu, const uint8_t* modes, void* ws, uint16_t* o, float* lse,
                         hipStream_t st) {
  DecArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.modes = modes;
  a.part = (float*)ws;
  a.nseq = d.nseq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.maxL = d.maxL;
  a.sink = d.sink;
  a.window = d.window;
  a.nsplit_max = decode_splits(d);
  a.c2 = d.scale * LOG2E;
  if (a.nsplit_max > 0) {
    const dim3 grid((unsigned)a.nsplit_max, (unsigned)d.Hkv, (unsigned)d.nseq);
    const int hpw = (d.G + 3) / 4;  // q-heads per wave: 1, 2, 3 or 4
    void (*kern)(DecArgs) = nullptr;
    if (d.D == 128) kern = hpw == 1 ? k_decode<128, 1> : hpw == 2 ? k_decode<128, 2> : k_decode<128, 4>;
    else kern = hpw == 1 ? k_decode<64, 1> : hpw == 2 ? k_decode<64, 2> : k_decode<64, 4>;
    hipLaunchKernelGGL(kern, grid, dim3(DEC_NT), 0, st, a);
  }
  const dim3 cgrid((unsigned)d.Hq, (unsigned)d.nseq);
  if (d.D == 128) hipLaunchKernelGGL(k_decode_combine<128>, cgrid, dim3(64), 0, st, a, o, lse);
  else hipLaunchKernelGGL(k_decode_combine<64>, cgrid, dim3(64), 0, st, a, o, lse);
  return hipGetLastError();
}

}  // namespace ea
