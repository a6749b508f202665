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
//   * split-K over waves: one wave takes a split of 256 to 4096 kept-key
//     positions of one (sequence, KV head) for
//     GW of its q-heads (all G when G <= 8), so each
//     K/V row is read once per GW heads.  The key set is compressed: an SSA
//     head's first split covers the sink and the start of the window.
//     The split length comes from the kept keys of the whole step: when the
//     modes could change it, a one-workgroup plan kernel sums them, picks
//     the split and lists the waves that have work, so a step whose heads
//     are mostly SSA still spreads over as many waves as an all-FA one, and
//     no idle wave sits between busy ones in the grid (the rest of the grid,
//     sized for the shortest split, ends at once).  Waves are independent:
//     no LDS staging and no workgroup barrier;
//   * lane layout: a key row of d bf16 is spread over d / 8 lanes, 16 bytes
//     each, so one wave load moves 64 / (d / 8) whole rows (contiguous 2 d
//     bytes per row) of K and of V;
//   * latency: K and V of three blocks of 4 iterations sit in a register
//     ring, two blocks in flight while one is computed;
//   * q . k: 4 v_dot2_f32_bf16 per lane and head, then a sum over the row's
//     lanes with DPP (quad swaps and row mirrors); exact online softmax per
//     block in the exp2 domain; P is rounded to bf16 and P V uses one
//     v_dot2_f32_bf16 per pair of iterations and column (the pairs built
//     with v_perm_b32), while the row sum stays in fp32;
//   * each wave writes (m, l, unnormalised o) of its split in fp32; a second
//     kernel combines the splits of every (sequence, q-head) into o (bf16)
//     and lse (fp32).
#include "ea_device.h"

namespace ea {

constexpr int DEC_BI = 4;   // iterations per softmax block
constexpr int DEC_NB = 3;   // blocks in the register ring

struct DecArgs {
  const uint16_t* q;   // [nseq, Hq, D]
  const uint16_t* k;   // [T, Hkv, D]
  const uint16_t* v;
  const int32_t* cu;
  const uint8_t* modes;
  float* part;         // [nseq, Hq, nsplit_max, D + 2]
  const int32_t* plan;  // null: split is fixed; else [0] split, [1] listed waves
  const int2* wlist;    // (unit, split) per listed wave, unit = (b Hkv + g) (G / GW) + wg
  // Segmented cache (null: k / v are the packed [T, Hkv, D] cache): rows of
  // (sequence b, KV head g) are [seg[b Hkv + g], seg[b Hkv + g + 1]) of a
  // head-major [cache_rows, D] pool; an SSA segment is a ring of its sink and
  // window keys (key j >= sink in slot sink + (j - sink) mod window).
  const int64_t* seg;
  int64_t cache_rows;
  int32_t nseq, Hq, Hkv, G, T, maxL, sink, window, split, nsplit_max;
  float c2;            // softmax scale * log2(e)
};

// Ring slot of key j >= sink of an SSA segment.
__device__ inline int64_t ring_slot(int64_t j, int32_t sink, int32_t window) {
  return (int64_t)sink + (j - sink) % window;
}

// Rows [lo, lo + cap) of unit i = b Hkv + g, clamped into the pool whatever
// the segment table holds; `last` is the last row a read may use (inside the
// segment, or a pool row if the segment is empty).
__device__ inline void seg_bounds(const DecArgs& a, int64_t i, int64_t* lo, int64_t* cap,
                                  int64_t* last) {
  const int64_t r = a.cache_rows;
  const int64_t s0 = min(max(a.seg[i], (int64_t)0), r);
  const int64_t s1 = min(max(a.seg[i + 1], s0), r);
  *lo = s0;
  *cap = s1 - s0;
  *last = s1 > s0 ? s1 - 1 : min(s0, r - 1);
}

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

// Sum over the LPK lanes that hold one key row (LPK = 8 or 16, aligned).
template <int LPK>
__device__ inline float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));  // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));  // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false)); // half-row mirror
  if (LPK == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));  // row mirror
  return x;
}

// Max / sum over the key groups of the wave (lanes LPK, 2 LPK, ... apart).
template <int LPK>
__device__ inline float groups_max(float x) {
  if (LPK == 8)
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));  // row_ror:8
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return halves_max(x);
}
template <int LPK>
__device__ inline float groups_sum(float x) {
  if (LPK == 8)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return halves_sum(x);
}

__device__ inline int32_t dec_split(const DecArgs& a) { return a.plan ? a.plan[0] : a.split; }

// Kept keys of (sequence, KV head) i = b * Hkv + g.
__device__ inline int32_t dec_kept_at(const DecArgs& a, int64_t i) {
  int32_t s0, L;
  seq_bounds(a, (int)(i / a.Hkv), &s0, &L);
  int mode = sane_mode(a.modes[i]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  return dec_kept(mode, L, a.sink, a.window);
}

// Plan of one decode step, one workgroup: the split (decode_split_rule over
// the kept keys of every (sequence, KV head) times the nwg head groups, no
// lower than s_min), then one wlist entry per wave that has work, units in
// order, so those waves are a prefix of the grid.  plan[0] = split,
// plan[1] = listed waves.  The list holds at most (units) * ceil(maxL /
// s_min) entries, the grid's size.
__global__ __launch_bounds__(1024) void k_decode_plan(DecArgs a, int32_t s_min, int32_t nwg,
                                                      int32_t* plan, int2* wlist) {
  __shared__ long long red[16];
  __shared__ int32_t wsum[16];
  __shared__ int32_t s_split;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t nbg = (int64_t)a.nseq * a.Hkv;
  long long w = 0;
  for (int64_t i = tid; i < nbg; i += 1024) w += dec_kept_at(a, i);
  for (int off = 32; off > 0; off >>= 1) w += __shfl_xor(w, off);
  if (lane == 0) red[wv] = w;
  __syncthreads();
  if (tid == 0) {
    long long t = 0;
    for (int i = 0; i < 16; ++i) t += red[i];
    s_split = decode_split_rule((int64_t)t * nwg, s_min);
  }
  __syncthreads();
  const int32_t S = s_split;
  // Exclusive scan of the per-unit split counts, 1024 units at a time.
  const int64_t nu = nbg * nwg;
  int32_t base = 0;
  for (int64_t c0 = 0; c0 < nu; c0 += 1024) {
    const int64_t u = c0 + tid;
    const int32_t cnt = u < nu ? cdiv(dec_kept_at(a, u / nwg), S) : 0;
    int32_t x = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int32_t before = 0, total = 0;
    for (int i = 0; i < 16; ++i) {
      const int32_t v = wsum[i];
      before += i < wv ? v : 0;
      total += v;
    }
    const int32_t first = base + before + x - cnt;
    for (int32_t j = 0; j < cnt; ++j) wlist[first + j] = make_int2((int)u, j);
    base += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) {
    plan[0] = S;
    plan[1] = base;
  }
}

template <int D, int GW, bool SEG>
__global__ __launch_bounds__(256) void k_decode(DecArgs a) {
  constexpr int LPK = D / 8;          // lanes per key row
  constexpr int KPI = 64 / LPK;       // keys per wave iteration
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPK, pc = lane % LPK;
  // Wave -> (split, head group, KV head, sequence): from the plan's list,
  // else split fastest.
  const int nwg = a.G / GW;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int32_t S, split;
  int64_t u;
  if (a.plan) {
    S = a.plan[0];
    if (w >= a.plan[1]) return;  // wave-uniform
    const int2 e = a.wlist[w];
    u = e.x;
    split = e.y;
  } else {
    S = a.split;
    split = (int)(w % a.nsplit_max);
    u = w / a.nsplit_max;
  }
  const int wg = (int)(u % nwg);
  u /= nwg;
  const int g = (int)(u % a.Hkv);
  const int b = (int)(u / a.Hkv);
  if (b >= a.nseq) return;
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  int mode = sane_mode(a.modes[(size_t)b * a.Hkv + g]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  const int32_t p0 = split * S;
  if (p0 >= n) return;  // wave-uniform
  const int32_t p1 = p0 + min(S, n - p0);
  const int nit = (p1 - p0 + KPI - 1) / KPI;
  const int nblk = (nit + DEC_BI - 1) / DEC_BI;
  const int h0 = g * a.G + wg * GW;

  // This lane's 16-byte piece of each of the GW queries.
  uint32_t qw[GW][4];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    const uint4 t = *(const uint4*)(a.q + ((size_t)b * a.Hq + h0 + hh) * D + 8 * pc);
    qw[hh][0] = t.x; qw[hh][1] = t.y; qw[hh][2] = t.z; qw[hh][3] = t.w;
  }

  // Segmented cache: this unit's rows, and for an SSA ring the slot of its
  // first window key (the window keys follow in slot order, wrapping once).
  int64_t seg_lo = 0, seg_last = 0, wslot0 = 0, ring_end = 0;
  int32_t head = 0;
  if (SEG) {
    int64_t seg_cap;
    seg_bounds(a, (int64_t)b * a.Hkv + g, &seg_lo, &seg_cap, &seg_last);
    head = min(a.sink, L);
    const int32_t jw0 = max(head, L - a.window);
    wslot0 = jw0 >= a.sink ? ring_slot(jw0, a.sink, a.window) : jw0;
    ring_end = (int64_t)a.sink + a.window;
  }
  uint4 kr[DEC_NB][DEC_BI], vr[DEC_NB][DEC_BI];
  auto load_block = [&](int blk, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int i = 0; i < DEC_BI; ++i) {
      const int32_t p = min(p0 + (blk * DEC_BI + i) * KPI + grp, p1 - 1);
      size_t off;
      if (SEG) {
        int64_t r = p;
        if (mode == EA_MODE_SSA && p >= head) {
          r = wslot0 + (p - head);
          if (r >= ring_end) r -= a.window;
        }
        off = (size_t)min(seg_lo + r, seg_last) * D + 8 * pc;
      } else {
        const int32_t j = dec_key(mode, p, L, a.sink, a.window);
        off = ((size_t)(s0 + j) * a.Hkv + g) * D + 8 * pc;
      }
      kr[sl][i] = *(const uint4*)(a.k + off);
      vr[sl][i] = *(const uint4*)(a.v + off);
    }
  };

  float m[GW], l[GW], o[GW][8];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[hh][c] = 0.f;
  }

  auto compute_block = [&](int blk, auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
    bool valid[DEC_BI];
#pragma unroll
    for (int i = 0; i < DEC_BI; ++i) valid[i] = p0 + (blk * DEC_BI + i) * KPI + grp < p1;
    // V of iteration pairs as (v_i[col], v_{i+1}[col]) words.
    uint32_t vp[DEC_BI / 2][8];
#pragma unroll
    for (int i = 0; i < DEC_BI; i += 2) {
      const uint32_t x[4] = {vr[sl][i].x, vr[sl][i].y, vr[sl][i].z, vr[sl][i].w};
      const uint32_t y[4] = {vr[sl][i + 1].x, vr[sl][i + 1].y, vr[sl][i + 1].z, vr[sl][i + 1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vp[i / 2][2 * e] = __builtin_amdgcn_perm(y[e], x[e], 0x05040100u);
        vp[i / 2][2 * e + 1] = __builtin_amdgcn_perm(y[e], x[e], 0x07060302u);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      float x[DEC_BI];
#pragma unroll
      for (int i = 0; i < DEC_BI; ++i) {
        const uint32_t kw[4] = {kr[sl][i].x, kr[sl][i].y, kr[sl][i].z, kr[sl][i].w};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]),
                                               __builtin_bit_cast(bf16x2, qw[hh][e]), acc, false);
        acc = row_sum<LPK>(acc);
        x[i] = valid[i] ? acc * a.c2 : -INFINITY;
      }
      float bm = x[0];
#pragma unroll
      for (int i = 1; i < DEC_BI; ++i) bm = fmaxf(bm, x[i]);
      const float mn = fmaxf(m[hh], groups_max<LPK>(bm));
      const float alpha = __builtin_amdgcn_exp2f(m[hh] - mn);  // m = -inf at the start: 0
      m[hh] = mn;
      float pf[DEC_BI], ps = 0.f;
#pragma unroll
      for (int i = 0; i < DEC_BI; ++i) {
        pf[i] = __builtin_amdgcn_exp2f(x[i] - mn);
        ps += pf[i];
      }
      l[hh] = l[hh] * alpha + ps;  // this key group's keys; groups are summed at the end
#pragma unroll
      for (int c = 0; c < 8; ++c) o[hh][c] *= alpha;
#pragma unroll
      for (int i = 0; i < DEC_BI; i += 2) {
        const bf16x2 pp = {(__bf16)pf[i], (__bf16)pf[i + 1]};
#pragma unroll
        for (int c = 0; c < 8; ++c)
          o[hh][c] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2, vp[i / 2][c]), o[hh][c],
                                                     false);
      }
    }
  };

  // Block blk lives in ring slot blk % 3; the body is unrolled three times so
  // that slots are compile-time register sets.
  load_block(0, std::integral_constant<int, 0>());
  if (nblk > 1) load_block(1, std::integral_constant<int, 1>());
  auto body = [&](int blk, auto slot_c, auto next_c) {
    if (blk + 2 < nblk) load_block(blk + 2, next_c);
    compute_block(blk, slot_c);
  };
  for (int blk = 0; blk < nblk; blk += DEC_NB) {
    body(blk, std::integral_constant<int, 0>(), std::integral_constant<int, 2>());
    if (blk + 1 < nblk) body(blk + 1, std::integral_constant<int, 1>(), std::integral_constant<int, 0>());
    if (blk + 2 < nblk) body(blk + 2, std::integral_constant<int, 2>(), std::integral_constant<int, 1>());
  }

  // Sum the key groups (m is already wave-uniform) and write the split.
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    const float lt = groups_sum<LPK>(l[hh]);
    float* dst = a.part + (((size_t)b * a.Hq + h0 + hh) * a.nsplit_max + split) * (D + 2);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float oc = groups_sum<LPK>(o[hh][c]);
      if (grp == 0) dst[8 * pc + c] = oc;
    }
    if (lane == 0) {
      dst[D] = m[hh];
      dst[D + 1] = lt;
    }
  }
}

// Combine the splits of one (sequence, q-head).  256 threads: the split
// maxima are reduced over the workgroup; then wave w folds splits w, w + 4,
// ... (lanes own CPL columns, loads of several splits in flight) and the
// four waves meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void k_decode_combine(DecArgs a, uint16_t* out, float* lse) {
  constexpr int CPL = D / 64;
  __shared__ float red[4 * (D + 2)];
  __shared__ float mred[4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  int mode = sane_mode(a.modes[(size_t)b * a.Hkv + h / a.G]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  const int32_t S = dec_split(a);
  const int ns = cdiv(n, S);
  const float* src = a.part + ((size_t)b * a.Hq + h) * a.nsplit_max * (D + 2);
  float M = -INFINITY;
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, src[(size_t)s * (D + 2) + D]);
  M = wave_max(M);
  if (lane == 0) mred[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(mred[0], mred[1]), fmaxf(mred[2], mred[3]));
  float Ls = 0.f, acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll 4
  for (int s = wv; s < ns; s += 4) {
    const float* row = src + (size_t)s * (D + 2);
    const float w = __builtin_amdgcn_exp2f(row[D] - M);
    Ls += w * row[D + 1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] += w * row[CPL * lane + c];
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) red[wv * (D + 2) + CPL * lane + c] = acc[c];
  if (lane == 0) red[wv * (D + 2) + D] = Ls;
  __syncthreads();
  if (wv == 0) {
    const float Lt = red[D] + red[(D + 2) + D] + red[2 * (D + 2) + D] + red[3 * (D + 2) + D];
    uint16_t* orow = out + ((size_t)b * a.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = CPL * lane + c;
      const float v = red[col] + red[(D + 2) + col] + red[2 * (D + 2) + col] + red[3 * (D + 2) + col];
      orow[col] = __builtin_bit_cast(uint16_t, (__bf16)(ns > 0 ? v / Lt : 0.f));
    }
    if (lane == 0) lse[(size_t)b * a.Hq + h] = ns > 0 ? (M + __log2f(Lt)) * LN2 : -INFINITY;
  }
}

// ------------------------------------------------------- segmented cache
// Fill: every kept key of every (sequence, KV head) of a packed [T, Hkv, D]
// k / v (e.g. the prefill's) into its segment row; one block covers RPB key
// positions of one unit, 16 bytes per thread.
template <int D>
__global__ __launch_bounds__(256) void k_cache_fill(DecArgs a, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v,
                                                    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  constexpr int CPR = D / 8, RPB = 256 / CPR;
  const int64_t unit = blockIdx.y;
  const int b = (int)(unit / a.Hkv), g = (int)(unit % a.Hkv);
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  int mode = sane_mode(a.modes[unit]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  int64_t lo, cap, last;
  seg_bounds(a, unit, &lo, &cap, &last);
  const int32_t p = (int32_t)blockIdx.x * RPB + (int32_t)(threadIdx.x / CPR);
  const int c = threadIdx.x % CPR;
  if (p >= n) return;
  const int32_t j = dec_key(mode, p, L, a.sink, a.window);
  const int64_t r = (mode == EA_MODE_SSA && j >= a.sink) ? ring_slot(j, a.sink, a.window) : j;
  if (r >= cap) return;
  const size_t src = ((size_t)(s0 + j) * a.Hkv + g) * D + 8 * c;
  const size_t dst = (size_t)(lo + r) * D + 8 * c;
  *(uint4*)(kc + dst) = *(const uint4*)(k + src);
  *(uint4*)(vc + dst) = *(const uint4*)(v + src);
}

// Append: the newest token (index L - 1 of each sequence, L from
// cu_seqlens) of every KV head, from k_new / v_new [nseq, Hkv, D], into its
// row or ring slot.
template <int D>
__global__ __launch_bounds__(256) void k_cache_append(DecArgs a, const uint16_t* __restrict__ kn,
                                                      const uint16_t* __restrict__ vn,
                                                      uint16_t* __restrict__ kc, uint16_t* __restrict__ vc) {
  constexpr int CPR = D / 8, UPB = 256 / CPR;
  const int64_t unit = (int64_t)blockIdx.x * UPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  if (unit >= (int64_t)a.nseq * a.Hkv) return;
  const int b = (int)(unit / a.Hkv);
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  if (L <= 0) return;
  const int mode = sane_mode(a.modes[unit]);
  const int64_t j = L - 1;
  const int64_t r = (mode == EA_MODE_SSA && j >= a.sink) ? ring_slot(j, a.sink, a.window) : j;
  int64_t lo, cap, last;
  seg_bounds(a, unit, &lo, &cap, &last);
  if (r >= cap) return;
  const size_t dst = (size_t)(lo + r) * D + 8 * c;
  const size_t src = (size_t)unit * D + 8 * c;
  *(uint4*)(kc + dst) = *(const uint4*)(kn + src);
  *(uint4*)(vc + dst) = *(const uint4*)(vn + src);
}

static DecArgs cache_args(const EaDims& d, const int32_t* cu, const uint8_t* modes, const int64_t* seg,
                          int64_t cache_rows) {
  DecArgs a = {};
  a.cu = cu;
  a.modes = modes;
  a.seg = seg;
  a.cache_rows = cache_rows;
  a.nseq = d.nseq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.maxL = d.maxL;
  a.sink = d.sink;
  a.window = d.window;
  return a;
}

hipError_t launch_cache_fill(const EaDims& d, const uint16_t* k, const uint16_t* v, const int32_t* cu,
                             const uint8_t* modes, const int64_t* seg, int64_t cache_rows,
                             uint16_t* kc, uint16_t* vc, hipStream_t st) {
  const DecArgs a = cache_args(d, cu, modes, seg, cache_rows);
  const int rpb = 256 / (d.D / 8);
  const dim3 grid((unsigned)cdiv(d.maxL, rpb), (unsigned)((int64_t)d.nseq * d.Hkv));
  if (d.D == 128) hipLaunchKernelGGL(k_cache_fill<128>, grid, dim3(256), 0, st, a, k, v, kc, vc);
  else hipLaunchKernelGGL(k_cache_fill<64>, grid, dim3(256), 0, st, a, k, v, kc, vc);
  return hipGetLastError();
}

hipError_t launch_cache_append(const EaDims& d, const uint16_t* kn, const uint16_t* vn, const int32_t* cu,
                               const uint8_t* modes, const int64_t* seg, int64_t cache_rows,
                               uint16_t* kc, uint16_t* vc, hipStream_t st) {
  const DecArgs a = cache_args(d, cu, modes, seg, cache_rows);
  const int upb = 256 / (d.D / 8);
  const dim3 grid((unsigned)(((int64_t)d.nseq * d.Hkv + upb - 1) / upb));
  if (d.D == 128) hipLaunchKernelGGL(k_cache_append<128>, grid, dim3(256), 0, st, a, kn, vn, kc, vc);
  else hipLaunchKernelGGL(k_cache_append<64>, grid, dim3(256), 0, st, a, kn, vn, kc, vc);
  return hipGetLastError();
}

hipError_t launch_decode(const EaDims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* cu, const uint8_t* modes, void* ws, const WsLayout& L,
                         uint16_t* o, float* lse, hipStream_t st, const int64_t* seg,
                         int64_t cache_rows) {
  DecArgs a = {};
  a.seg = seg;
  a.cache_rows = cache_rows;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.modes = modes;
  a.part = (float*)((char*)ws + L.dec_part);
  a.nseq = d.nseq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.maxL = d.maxL;
  a.sink = d.sink;
  a.window = d.window;
  // Splits of at least decode_split_min: the partials hold nsplit_max of them
  // per (sequence, q-head) and the grid one wave each.
  const int gw = decode_gw(d);
  a.split = decode_split_min(d);
  a.nsplit_max = decode_splits(d);
  a.plan = nullptr;
  a.wlist = nullptr;
  a.c2 = d.scale * LOG2E;
  if (a.nsplit_max > 0 && decode_split_max(d) > a.split) {
    int32_t* plan = (int32_t*)((char*)ws + L.dec_plan);
    int2* wlist = (int2*)((char*)ws + L.dec_waves);
    hipLaunchKernelGGL(k_decode_plan, dim3(1), dim3(1024), 0, st, a, a.split, d.G / gw, plan, wlist);
    a.plan = plan;
    a.wlist = wlist;
  }
  if (a.nsplit_max > 0) {
    const int64_t waves = decode_waves(d);
    const dim3 grid((unsigned)((waves + 3) / 4));
    void (*kern)(DecArgs) = nullptr;
    if (seg) {
      if (d.D == 128)
        kern = gw == 8 ? k_decode<128, 8, true> : gw == 4 ? k_decode<128, 4, true>
             : gw == 2 ? k_decode<128, 2, true> : k_decode<128, 1, true>;
      else
        kern = gw == 8 ? k_decode<64, 8, true> : gw == 4 ? k_decode<64, 4, true>
             : gw == 2 ? k_decode<64, 2, true> : k_decode<64, 1, true>;
    } else {
      if (d.D == 128)
        kern = gw == 8 ? k_decode<128, 8, false> : gw == 4 ? k_decode<128, 4, false>
             : gw == 2 ? k_decode<128, 2, false> : k_decode<128, 1, false>;
      else
        kern = gw == 8 ? k_decode<64, 8, false> : gw == 4 ? k_decode<64, 4, false>
             : gw == 2 ? k_decode<64, 2, false> : k_decode<64, 1, false>;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a);
  }
  const dim3 cgrid((unsigned)d.Hq, (unsigned)d.nseq);
  if (d.D == 128) hipLaunchKernelGGL(k_decode_combine<128>, cgrid, dim3(256), 0, st, a, o, lse);
  else hipLaunchKernelGGL(k_decode_combine<64>, cgrid, dim3(256), 0, st, a, o, lse);
  return hipGetLastError();
}

}  // namespace ea
