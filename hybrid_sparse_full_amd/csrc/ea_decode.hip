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
//   * split-K over waves: one wave takes a split of 64 to 4096 kept-key
//     positions of one (sequence, KV head) for
//     GW of its q-heads (all G when G <= 8), so each
//     K/V row is read once per GW heads.  The key set is compressed: an SSA
//     head's first split covers the sink and the start of the window.
//     The split length comes from the kept keys of the whole step: when the
//     modes could change it, a one-workgroup plan kernel sums them, picks
//     the split and lists the workgroups that have work, so a step whose
//     heads are mostly SSA still spreads over as many waves as an all-FA
//     one, and no idle workgroup sits between busy ones in the grid (the
//     rest of the grid, sized for the shortest split, ends at once).  The
//     DEC_WPG waves of a workgroup take consecutive splits of one
//     (sequence, KV head, head group); they stream their keys independently
//     and meet once, at the end, to merge their results in LDS;
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
//   * each workgroup writes one partial (m, l, unnormalised o) in fp32 for
//     each of its heads; a second kernel combines the partials of every
//     (sequence, q-head) into o (bf16) and lse (fp32) in one online pass,
//     with the 16-byte loads of many partials in flight per thread.
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
  float* part;         // unnormalised o of each partial: [nseq, Hq, nparts, D]
  float2* ml;          // (m, l) of each partial: [nseq, Hq, nparts]
  const int32_t* plan;  // null: split is fixed; else [0] split, [1] listed workgroups
  const int2* glist;    // (unit, partial) per listed workgroup, unit = (b Hkv + g) (G / GW) + wg
  // Plan inside k_decode (few units): split = rule over the kept keys, no
  // lower than `split`; workgroup 0 stores it in plan_out[0] for the combine.
  int32_t* plan_out;
  int32_t inline_plan;
  // Segmented cache (null: k / v are the packed [T, Hkv, D] cache): rows of
  // (sequence b, KV head g) are [seg[b Hkv + g], seg[b Hkv + g + 1]) of a
  // head-major [cache_rows, D] pool; an SSA segment is a ring of its sink and
  // window keys (key j >= sink in slot sink + (j - sink) mod window).
  const int64_t* seg;
  int64_t cache_rows;
  int32_t nseq, Hq, Hkv, G, T, maxL, sink, window, split, nparts;
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
  const int32_t e = (int32_t)min<int64_t>(min(max(a.cu[b + 1], s), a.T), (int64_t)s + a.maxL);
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
// lower than s_min), then one glist entry per workgroup that has work (a
// workgroup covers DEC_WPG splits), units in order, so those workgroups are
// a prefix of the grid.  plan[0] = split, plan[1] = listed workgroups.  The
// list holds at most (units) * cdiv(maxL, DEC_WPG * s_min) entries, the
// grid's size.  Units are taken 1024 at a time: a block scan of their
// workgroup counts gives each unit its first entry, then every thread fills
// entries and finds an entry's unit by binary search over those firsts.
__global__ __launch_bounds__(1024) void k_decode_plan(DecArgs a, int32_t s_min, int32_t nwg,
                                                      int32_t* plan, int2* glist) {
  __shared__ long long red[16];
  __shared__ int32_t wsum[16];
  __shared__ int32_t s_split;
  __shared__ int32_t first[1024];
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
  const int64_t per = (int64_t)DEC_WPG * S;  // kept keys per workgroup
  const int64_t nu = nbg * nwg;
  int32_t base = 0;
  for (int64_t c0 = 0; c0 < nu; c0 += 1024) {
    const int64_t u = c0 + tid;
    const int32_t cnt = u < nu ? (int32_t)((dec_kept_at(a, u / nwg) + per - 1) / per) : 0;
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
    first[tid] = base + before + x - cnt;
    __syncthreads();
    // Entry e of this chunk belongs to its last unit whose first entry is at
    // most e (a unit with no workgroups shares its first with the next one).
    const int nloc = (int)(nu - c0 < 1024 ? nu - c0 : 1024);
    for (int32_t e = base + tid; e < base + total; e += 1024) {
      const int i = upper_index(first, nloc, e);
      glist[e] = make_int2((int)(c0 + i), e - first[i]);
    }
    base += total;
    __syncthreads();  // first and wsum are rewritten by the next chunk
  }
  if (tid == 0) {
    plan[0] = S;
    plan[1] = base;
  }
}

template <int D, int GW, bool SEG>
__global__ __launch_bounds__(DEC_WPG * 64) void k_decode(DecArgs a) {
  constexpr int LPK = D / 8;          // lanes per key row
  constexpr int KPI = 64 / LPK;       // keys per wave iteration
  constexpr int CPL = D / 64;         // merged columns per lane
  // Each wave's (o, m, l) per head, merged once all waves are done.
  __shared__ float red[DEC_WPG][GW][D + 2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int grp = lane / LPK, pc = lane % LPK;
  // Workgroup -> (partial, head group, KV head, sequence): from the plan's
  // list, else partial fastest.  Every early return below is uniform over
  // the workgroup, so all its waves reach the merge barrier.
  const int nwg = a.G / GW;
  int32_t S, part, s0, L;
  int64_t u;
  int mode;
  if (a.inline_plan) {
    // Lane i holds unit i (at most 64 units): its sequence bounds, mode and
    // workgroup count; the workgroup's unit is the number of units whose
    // inclusive count is at most blockIdx.x.
    const int nu = a.nseq * a.Hkv * nwg;
    int64_t kept = 0;
    int32_t us0 = 0, uL = 0, um = EA_MODE_FA;
    if (lane < nu) {
      const int bg = lane / nwg;
      seq_bounds(a, bg / a.Hkv, &us0, &uL);
      um = sane_mode(a.modes[bg]);
      if (um == EA_MODE_XA) um = EA_MODE_FA;
      kept = dec_kept(um, uL, a.sink, a.window);
    }
    S = decode_split_rule(wave_sum(kept), a.split);
    if (blockIdx.x == 0 && threadIdx.x == 0) a.plan_out[0] = S;
    const int64_t per = (int64_t)DEC_WPG * S;
    const int32_t cnt = (int32_t)((kept + per - 1) / per);
    const int32_t incl = wave_inclusive_sum(cnt);
    if ((int)blockIdx.x >= __shfl(incl, 63)) return;
    const int ui = __popcll(__ballot(incl <= (int)blockIdx.x));
    part = (int)blockIdx.x - (__shfl(incl, ui) - __shfl(cnt, ui));
    u = ui;
    s0 = __shfl(us0, ui);
    L = __shfl(uL, ui);
    mode = __shfl(um, ui);
  } else {
    if (a.plan) {
      S = a.plan[0];
      if ((int64_t)blockIdx.x >= a.plan[1]) return;
      const int2 e = a.glist[blockIdx.x];
      u = e.x;
      part = e.y;
    } else {
      S = a.split;
      part = (int)(blockIdx.x % a.nparts);
      u = blockIdx.x / a.nparts;
    }
    const int b = (int)(u / nwg / a.Hkv);
    if (b >= a.nseq) return;
    seq_bounds(a, b, &s0, &L);
    mode = sane_mode(a.modes[(size_t)(u / nwg)]);
    if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  }
  const int wg = (int)(u % nwg);
  u /= nwg;
  const int g = (int)(u % a.Hkv);
  const int b = (int)(u / a.Hkv);
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  const int64_t gbase = (int64_t)part * DEC_WPG * S;
  if (gbase >= n) return;  // no partial of this workgroup is combined
  // This wave's split; the last waves of a unit's last workgroup may get none.
  const int32_t p0 = (int32_t)min<int64_t>(gbase + (int64_t)wv * S, n);
  const int32_t p1 = (int32_t)min<int64_t>((int64_t)p0 + S, n);
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
  if (nblk > 0) load_block(0, std::integral_constant<int, 0>());
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

  // Sum the key groups (m is already wave-uniform) and stage the split's
  // result; a wave without keys stages m = -inf, l = 0, o = 0.
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    const float lt = groups_sum<LPK>(l[hh]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float oc = groups_sum<LPK>(o[hh][c]);
      if (grp == 0) red[wv][hh][8 * pc + c] = oc;
    }
    if (lane == 0) {
      red[wv][hh][D] = m[hh];
      red[wv][hh][D + 1] = lt;
    }
  }
  __syncthreads();
  // Merge the workgroup's splits (wave w takes heads w, w + DEC_WPG, ...)
  // into one partial; wave 0's split has keys, so M is finite.
  for (int hh = wv; hh < GW; hh += DEC_WPG) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < DEC_WPG; ++i) M = fmaxf(M, red[i][hh][D]);
    float Ls = 0.f, acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < DEC_WPG; ++i) {
      const float mi = red[i][hh][D];
      const float wt = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - M);
      Ls += wt * red[i][hh][D + 1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += wt * red[i][hh][CPL * lane + c];
    }
    const size_t idx = ((size_t)b * a.Hq + h0 + hh) * a.nparts + part;
#pragma unroll
    for (int c = 0; c < CPL; ++c) a.part[idx * D + CPL * lane + c] = acc[c];
    if (lane == 0) a.ml[idx] = make_float2(M, Ls);
  }
}

// Combine the partials of one (sequence, q-head) in one online pass.  512
// threads: a partial's o row is read by D / 4 threads (16 bytes each), so
// 512 / (D / 4) partials are read side by side, and each thread issues the
// loads of U of its partials before it uses any; each thread keeps a
// running (m, l, o) over its partials, rescaled once per batch, and the
// thread groups meet in LDS at the end.
template <int D>
__global__ __launch_bounds__(512) void k_decode_combine(DecArgs a, uint16_t* out, float* lse) {
  constexpr int TPR = D / 4;     // threads per partial row
  constexpr int NGR = 512 / TPR; // partials side by side
  constexpr int U = 16;          // partials per thread per batch
  __shared__ float red[NGR][D + 2];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int gi = tid / TPR, j = tid % TPR;
  int32_t s0, L;
  seq_bounds(a, b, &s0, &L);
  int mode = sane_mode(a.modes[(size_t)b * a.Hkv + h / a.G]);
  if (mode == EA_MODE_XA) mode = EA_MODE_FA;
  const int32_t n = dec_kept(mode, L, a.sink, a.window);
  const int64_t per = (int64_t)DEC_WPG * dec_split(a);
  const int ns = (int)((n + per - 1) / per);
  const size_t row0 = ((size_t)b * a.Hq + h) * a.nparts;
  float m = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sb = gi; sb < ns; sb += NGR * U) {
    float2 ml[U];
    f32x4 ov[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int s = sb + k * NGR;
      if (s < ns) {
        ml[k] = a.ml[row0 + s];
        ov[k] = *(const f32x4*)(a.part + (row0 + s) * D + 4 * j);
      } else {
        ml[k] = make_float2(-INFINITY, 0.f);
        ov[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // Partial sb is inside [0, ns), so the batch maximum is finite.
    float mb = m;
#pragma unroll
    for (int k = 0; k < U; ++k) mb = fmaxf(mb, ml[k].x);
    const float sc = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mb);
    l *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float w = ml[k].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - mb);
      l += w * ml[k].y;
      acc += w * ov[k];
    }
    m = mb;
  }
  *(f32x4*)&red[gi][4 * j] = acc;
  if (j == 0) {
    red[gi][D] = m;
    red[gi][D + 1] = l;
  }
  __syncthreads();
  if (tid < TPR) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < NGR; ++g) M = fmaxf(M, red[g][D]);
    float Lt = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NGR; ++g) {
      const float mg = red[g][D];
      const float w = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg - M);
      Lt += w * red[g][D + 1];
      o += w * *(const f32x4*)&red[g][4 * tid];
    }
    const float inv = ns > 0 ? 1.0f / Lt : 0.f;
    const bf16x4 hv = __builtin_convertvector(o * inv, bf16x4);
    *(bf16x4*)(out + ((size_t)b * a.Hq + h) * D + 4 * tid) = hv;
    if (tid == 0) lse[(size_t)b * a.Hq + h] = ns > 0 ? (M + __log2f(Lt)) * LN2 : -INFINITY;
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
  a.ml = (float2*)((char*)ws + L.dec_ml);
  a.nseq = d.nseq;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.T = d.T;
  a.maxL = d.maxL;
  a.sink = d.sink;
  a.window = d.window;
  // Splits of at least decode_split_min: the partials hold nparts of them
  // per (sequence, q-head) and the grid one workgroup each.
  const int gw = decode_gw(d);
  a.split = decode_split_min(d);
  a.nparts = decode_parts(d);
  a.plan = nullptr;
  a.glist = nullptr;
  a.plan_out = nullptr;
  a.inline_plan = 0;
  a.c2 = d.scale * LOG2E;
  if (a.nparts > 0 && decode_split_max(d) > a.split) {
    int32_t* plan = (int32_t*)((char*)ws + L.dec_plan);
    if ((int64_t)d.nseq * d.Hkv * (d.G / gw) <= DEC_INLINE_UNITS) {
      a.inline_plan = 1;
      a.plan_out = plan;
    } else {
      int2* glist = (int2*)((char*)ws + L.dec_groups);
      hipLaunchKernelGGL(k_decode_plan, dim3(1), dim3(1024), 0, st, a, a.split, d.G / gw, plan, glist);
      a.glist = glist;
    }
    a.plan = plan;
  }
  if (a.nparts > 0) {
    const dim3 grid((unsigned)decode_groups(d));
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
    hipLaunchKernelGGL(kern, grid, dim3(DEC_WPG * 64), 0, st, a);
  }
  const dim3 cgrid((unsigned)d.Hq, (unsigned)d.nseq);
  if (d.D == 128) hipLaunchKernelGGL(k_decode_combine<128>, cgrid, dim3(512), 0, st, a, o, lse);
  else hipLaunchKernelGGL(k_decode_combine<64>, cgrid, dim3(512), 0, st, a, o, lse);
  return hipGetLastError();
}

}  // namespace ea
