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

__device__ inline int64_t tri_root(int64_t loc) {
  int64_t t = (int64_t)((sqrt(8.0 * (double)loc + 1.0) - 1.0) * 0.5);
  while (tri64(t + 1) <= loc) ++t;
  while (tri64(t) > loc) --t;
  return t;
}

// One scoring item is a 128 x 128 tile (reduced keys b' x reduced queries a)
// of a group of HPI q-heads that share one KV head: the K~ chunk of every
// stage is staged once and serves all HPI heads.  With GROUP (one mask per
// KV head, HPI == G) the 8 waves split one tile and each accumulates the
// products of all HPI heads into the same registers: the sum of the heads'
// scores, divided by HPI in the epilogue, is the group-mean score.
//
// A stage is KC = 64 elements of the S * d reduction (part of one key row t
// of the antidiagonal); the stages of an item stream through an LDS ring of
// NS slots by global->LDS DMA, NS - 1 stages ahead of the MFMAs (two 80 KB
// stages with four heads per item; measured: halving KC to keep a four-stage
// ring was 6 % slower, its extra barriers cost more than the deeper
// prefetch hid).  Rows of a staged tile are KC * 2 bytes, RPL = 256 / (KC * 2) of
// them share the 64 LDS banks; the 16-byte chunks of row r are XOR-swizzled
// by (r / RPL) % CPR, which puts the 16 rows that one 16-lane group of a
// 128-bit operand read touches on 16 distinct 4-bank groups (a swizzle by
// r % CPR alone gives rows r and r + CPR the same banks).
template <int D, int R, int HPI, bool GROUP = false>
struct XaCfg {
  static constexpr int NW = 8;                   // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int KC = 64;                  // reduction elements per stage
  static constexpr int ROWB = KC * 2;            // bytes per staged row
  static constexpr int CPR = KC / 8;             // 16-byte chunks per staged row
  static constexpr int RPL = 256 / ROWB;         // staged rows per 64-bank line
  static constexpr int RPG = 1024 / ROWB;        // staged rows per 1 KB DMA region
  static constexpr int OPB = XT * ROWB;          // one staged operand tile
  static constexpr int OPR = OPB / 1024;         // DMA regions per operand tile
  static constexpr int STAGE = (1 + HPI) * OPB;  // K~ then HPI Q~ tiles
  static constexpr int NS = HPI == 4 ? 2 : 3;    // stages in the LDS ring
  static constexpr int NI = STAGE / 1024 / NW;   // 1 KB DMA regions per wave per stage
  static constexpr int WPH = GROUP ? NW : NW / HPI;            // waves per output tile
  static constexpr int AW = (GROUP || HPI == 1) ? 4 : WPH;     // waves along a (queries)
  static constexpr int NHQ = GROUP ? HPI : 1;                  // heads summed by a wave
  static constexpr int BW = WPH / AW;            // waves along b' (keys)
  static constexpr int NA = XT / AW / 32;        // 32-query MFMA tiles per wave
  static constexpr int NB = XT / BW / 32;        // 32-key MFMA tiles per wave
  static constexpr int KSTEPS = KC / 16;
  static_assert((STAGE / 1024) % NW == 0, "DMA regions must split evenly over waves");
  static_assert(NS * STAGE <= 160 * 1024, "the ring must fit in LDS");
  static_assert((NS - 2) * NI <= 63, "vmcnt holds at most 63");
};

// Wait until this wave's DMA of the current stage has landed, with `ahead`
// later stages (at most NS - 2) allowed in flight, then join the barrier.
template <int NI, int NS>
__device__ inline void stage_wait(int ahead) {
  if constexpr (NS >= 4) {
    if (ahead >= 2) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(2 * NI) : "memory");
      return;
    }
  }
  if constexpr (NS >= 3) {
    if (ahead >= 1) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(NI) : "memory");
      return;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
}

template <int D, int R, int HPI, bool GROUP>
__global__ __launch_bounds__(512) void k_xa_score(EaDims d, const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k, SeqMeta m,
                                                  const int32_t* __restrict__ pair_bg,
                                                  const int64_t* __restrict__ pair_items,
                                                  float* __restrict__ lse_ws) {
  using C = XaCfg<D, R, HPI, GROUP>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::NS * C::STAGE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int hh = GROUP ? 0 : wv / C::WPH;          // head of the group (GROUP: all)
  const int wa = (wv % C::WPH) % C::AW, wb = (wv % C::WPH) / C::AW;
  const int npairs = m.scal[SCAL_XA_PAIRS];
  const int64_t total = pair_items[npairs];
  unsigned long long* ctr = (unsigned long long*)(m.scal + SCAL_CTR64);
  const float C2 = d.scale * LOG2E * (GROUP ? 1.0f / HPI : 1.0f);
  const float Cs = d.scale * (GROUP ? 1.0f / HPI : 1.0f);  // natural units (block sums)
  const bool raw_sums = d.xa_norm != 0;
  const int S = d.S;
  const int nhg = d.Hq / HPI;
  const int nst = S * D / C::KC;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // DMA: lane l of a 1 KB region (RPG staged rows) writes row l / CPR of the
  // region, physical chunk l % CPR, which holds logical chunk
  // (l % CPR) ^ ((row / RPL) % CPR).
  const int rr = lane / C::CPR;
  // MFMA operand reads: lane reads row 32 t + l32 at logical chunk 2 s + half,
  // physical chunk (2 s + half) ^ ((l32 / RPL) % CPR) (32 t / RPL is a
  // multiple of CPR); the 2 s part is XORed in per k-step.
  const uint32_t fa = (uint32_t)l32 * C::ROWB +
                      (((uint32_t)half ^ ((uint32_t)(l32 / C::RPL) % C::CPR)) << 4);
  volatile int64_t* item_box = (volatile int64_t*)smem;

  while (true) {
    __syncthreads();  // the previous item's readers are done with the ring
    if (tid == 0) *item_box = (int64_t)atomicAdd(ctr, 1ull);
    __syncthreads();
    const int64_t item = *item_box;
    __syncthreads();  // everyone has the item before the ring is refilled
    if (item >= total) break;
    const int p = upper_index(pair_items, npairs + 1, item);
    const int64_t loc = item - pair_items[p];
    const int64_t ta = tri_root(loc);
    const int64_t tb = loc - tri64(ta);
    const int32_t bg = pair_bg[p];
    const int b = bg / nhg, h0 = (bg % nhg) * HPI, g = h0 / d.G;
    const int64_t tok0 = m.start[b];
    const int32_t len = m.len[b];
    const int32_t nred = len / S;
    const int64_t nqb = len / d.B;
    const int32_t a0 = (int32_t)ta * XT, b0 = (int32_t)tb * XT;

    // Per-lane global address of each of this wave's DMA regions at t = 0,
    // dk = 0 (rows past the sequence end read its last reduced row; their
    // products are masked in the epilogue).
    uint64_t gaddr[C::NI];
    uint32_t gop[C::NI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int jj = wv * C::NI + i;
      const int op = jj / C::OPR, row = C::RPG * (jj % C::OPR) + rr;
      const int lch = (lane % C::CPR) ^ ((row / C::RPL) % C::CPR);
      gop[i] = (uint32_t)op;
      if (op == 0) {
        const int64_t bp = min(b0 + row, nred - 1);
        const int64_t tok = tok0 + bp * S + (S - 1);
        gaddr[i] = (uint64_t)(uintptr_t)(k + (tok * d.Hkv + g) * D + lch * 8);
      } else {
        const int64_t a = min(a0 + row, nred - 1);
        const int64_t tok = tok0 + a * S;
        gaddr[i] = (uint64_t)(uintptr_t)(q + (tok * d.Hq + h0 + op - 1) * D + lch * 8);
      }
    }
    // Stage st: t = st * KC / D, dk = st * KC % D; K~ walks t backwards.
    // DMA instruction i of this wave for stage st.
    auto issue_one = [&](int st, int i) __attribute__((always_inline)) {
      const int t = st * C::KC / D, dk = st * C::KC % D;
      const int64_t dK = ((int64_t)(-t) * d.Hkv * D + dk) * 2;
      const int64_t dQ = ((int64_t)t * d.Hq * D + dk) * 2;
      const uint32_t slot = lds0 + (uint32_t)(st % C::NS) * C::STAGE;
      const int jj = wv * C::NI + i;
      const uint64_t ga = gaddr[i] + (uint64_t)(gop[i] == 0 ? dK : dQ);
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(slot + (uint32_t)jj * 1024u);
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(ga), "s"(m0v)
                   : "m0");
    };
    auto issue = [&](int st) {
#pragma unroll
      for (int i = 0; i < C::NI; ++i) issue_one(st, i);
    };

    f32x16 acc[C::NA][C::NB];
#pragma unroll
    for (int i = 0; i < C::NA; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
    for (int s0 = 0; s0 < C::NS - 1; ++s0)
      if (s0 < nst) issue(s0);
    for (int st = 0; st < nst; ++st) {
      // Stage st has landed (own DMA) once at most the later stages' are in
      // flight; the barrier extends that to every wave and frees the slot
      // the next issue overwrites.
      stage_wait<C::NI, C::NS>(min(C::NS - 2, nst - 1 - st));
      // The DMA of stage st + NS - 1 goes out between this stage's first
      // MFMAs, one instruction after every second (measured 2 % faster than
      // issuing it in one burst before them, and than one per MFMA or per
      // three).  The DMA is the largest single cost of the item (about a
      // quarter of its time, growing with the bytes moved), ahead of the
      // epilogue (about a tenth).
      const bool dnext = st + C::NS - 1 < nst;
      const int snext = st + C::NS - 1;
      constexpr int MPS = C::KSTEPS * C::NHQ * C::NA * C::NB;  // MFMAs per stage
      constexpr int EVERY = 2;
      const uint32_t slot = (uint32_t)(st % C::NS) * C::STAGE;
      const uint8_t* Ks = smem + slot + (size_t)wb * (C::NB * 32) * C::ROWB;
      const uint8_t* Qs = smem + slot + (size_t)(1 + hh) * C::OPB + (size_t)wa * (C::NA * 32) * C::ROWB;
      auto kf = [&](int j, int s) { return *(const bf16x8*)(Ks + (fa ^ (uint32_t)(s << 5)) + j * 32 * C::ROWB); };
      auto qf = [&](int u, int i, int s) {
        return *(const bf16x8*)(Qs + (size_t)u * C::OPB + (fa ^ (uint32_t)(s << 5)) + i * 32 * C::ROWB);
      };
      bf16x8 fk[2][C::NB], fq[2][C::NHQ][C::NA];
#pragma unroll
      for (int j = 0; j < C::NB; ++j) fk[0][j] = kf(j, 0);
#pragma unroll
      for (int u = 0; u < C::NHQ; ++u)
#pragma unroll
        for (int i = 0; i < C::NA; ++i) fq[0][u][i] = qf(u, i, 0);
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        if (s + 1 < C::KSTEPS) {
#pragma unroll
          for (int j = 0; j < C::NB; ++j) fk[(s + 1) & 1][j] = kf(j, s + 1);
#pragma unroll
          for (int u = 0; u < C::NHQ; ++u)
#pragma unroll
            for (int i = 0; i < C::NA; ++i) fq[(s + 1) & 1][u][i] = qf(u, i, s + 1);
        }
#pragma unroll
        for (int u = 0; u < C::NHQ; ++u)
#pragma unroll
          for (int i = 0; i < C::NA; ++i)
#pragma unroll
            for (int j = 0; j < C::NB; ++j) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[s & 1][j], fq[s & 1][u][i], acc[i][j], 0, 0, 0);
              const int mi = ((s * C::NHQ + u) * C::NA + i) * C::NB + j;
              if (mi % EVERY == EVERY - 1 && mi / EVERY < C::NI) {
                __builtin_amdgcn_sched_barrier(0);
                if (dnext) issue_one(snext, mi / EVERY);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
      }
      // Instructions the interleave did not place (NI > MPS).
#pragma unroll
      for (int i = MPS / EVERY; i < C::NI; ++i)
        if (dnext) issue_one(snext, i);
    }

    // Epilogue: per (reduced row a, block J) log-sum-exp in log2 units.
    const int h = h0 + hh;
    const int64_t base_bh = (int64_t)R * (m.tri_prefix[b] * d.Hq + (int64_t)h * tri64(nqb));
    // Register r of a lane holds reduced key 8 (r >> 2) + 4 half + (r & 3) of
    // the 32-key MFMA tile.  With R >= 8 a block spans both half-waves (R / 2
    // registers per lane); with R == 4 it lies in one half-wave: registers
    // 4k..4k+3 of half h hold block 2k + h.
    constexpr int NG = R >= 8 ? 32 / R : 4;  // blocks per 32-key MFMA tile per lane
    constexpr int RPG = R >= 8 ? R / 2 : 4;  // registers per block per lane
    // A tile strictly below the diagonal block row and inside the sequence
    // needs neither the causal nor the range test.
    const bool interior = b0 + XT <= a0 && a0 + XT <= nred;
    auto epilogue = [&](auto full_c) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int i = 0; i < C::NA; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          const int32_t a = a0 + (wa * C::NA + i) * 32 + l32;
          const int32_t Ia = a / R;
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            const int32_t brow0 = b0 + (wb * C::NB + j) * 32 + (R >= 8 ? gi * R : 8 * gi + 4 * half);
            const int32_t J = brow0 / R;
            float v[RPG];
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < RPG; ++e) {
              const int r = gi * RPG + e;
              const int32_t bq = b0 + (wb * C::NB + j) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              const bool ok = FULL || ((bq <= a) && (a < nred));
              v[e] = ok ? acc[i][j][r] : -INFINITY;
              mloc = fmaxf(mloc, v[e]);
            }
            float out;
            if (__builtin_expect(raw_sums, 0)) {
              // Block-sum masses: the plain sum of the allowed scores.
              float sr = 0.f;
#pragma unroll
              for (int e = 0; e < RPG; ++e) sr += v[e] == -INFINITY ? 0.f : v[e];
              if (R >= 8) sr = halves_sum(sr);
              out = sr * Cs;
            } else {
              const float mm = R >= 8 ? halves_max(mloc) : mloc;
              float sum = 0.f;
              if (FULL || mm != -INFINITY) {
#pragma unroll
                for (int e = 0; e < RPG; ++e) sum += __builtin_amdgcn_exp2f((v[e] - mm) * C2);
              }
              if (R >= 8) sum = halves_sum(sum);
              out = mm * C2 + __builtin_amdgcn_logf(sum);
            }
            if ((R < 8 || half == 0) && (FULL || (a < nred && J <= Ia))) {
              const int64_t idx = base_bh + (int64_t)R * tri64(Ia) + (int64_t)(a - R * Ia) * (Ia + 1) + J;
              lse_ws[idx] = out;
            }
          }
        }
    };
    if (interior) epilogue(std::true_type());
    else epilogue(std::false_type());
  }
}

// ---------------------------------------------------------------- selector
// One wave per mask row (rows are independent, so no workgroup barrier is
// needed); each wave keeps the row's block masses, weights and bits in its
// own LDS region.

template <int R>
__global__ __launch_bounds__(256) void k_xa_select(EaDims d, const uint8_t* __restrict__ modes,
                                                   SeqMeta m, const float* __restrict__ lse_ws,
                                                   uint32_t* __restrict__ mask,
                                                   int32_t* __restrict__ row_count,
                                                   int64_t* __restrict__ xa_pairs,
                                                   float* __restrict__ block_mass) {
  extern __shared__ uint32_t dyn[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rpw = blockDim.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * rpw + wv;
  if (row >= d.nqb_max * d.Hq) return;
  const int32_t qbg = (int32_t)(row / d.Hq);
  const int h = (int)(row % d.Hq);
  uint32_t* mrow = mask + row * d.words;
  if (qbg >= m.scal[SCAL_TOTAL_QB]) {
    // Rows past the last q-block of the batch (the row count is a bound
    // from the descriptor): written as empty, like rows of non-XA heads.
    for (int w = lane; w < d.words; w += 64) mrow[w] = 0u;
    if (lane == 0) row_count[row] = 0;
    return;
  }
  uint32_t* wgt = dyn + (size_t)wv * (d.maxqb + d.words);
  uint32_t* bits = wgt + d.maxqb;
  const int32_t b = m.qb2seq[qbg];
  const int32_t I = qbg - m.qb_prefix[b];
  const int32_t len = m.len[b];
  const int mode = sane_mode(modes[(int64_t)b * d.Hkv + h / d.G]);
  const int32_t nI = I + 1;
  if (mode != EA_MODE_XA) {
    for (int w = lane; w < d.words; w += 64) mrow[w] = 0u;
    if (lane == 0) row_count[row] = 0;
    return;
  }
  const int64_t B = d.B;
  if (len % d.B != 0) {
    // XA on a sequence that is not a whole number of blocks: every causal block.
    for (int w = lane; w < d.words; w += 64) {
      const int hi = I - w * 32;
      mrow[w] = hi < 0 ? 0u : (hi >= 31 ? 0xffffffffu : ((2u << hi) - 1u));
    }
    if (lane == 0) {
      row_count[row] = nI;
      const int64_t iend = min<int64_t>((int64_t)nI * B, len);
      atomicAdd((unsigned long long*)&xa_pairs[(int64_t)b * d.Hq + h],
                (unsigned long long)(tri64(iend) - tri64((int64_t)I * B)));
    }
    return;
  }

  const int64_t nqb = len / d.B;
  // One mask per KV head: every q-head of the group reads the scores that the
  // group's first head slot holds.
  const int hs = d.xa_group ? h - h % d.G : h;
  const float* base =
      lse_ws + (int64_t)R * (m.tri_prefix[b] * d.Hq + (int64_t)hs * tri64(nqb)) + (int64_t)R * tri64(I);
  // 1. Per reduced row a: La = log2 sum_J exp2(lse2[a, J]), one online pass
  //    (lane-local running max and sum, then merged over the wave).  With
  //    block-sum masses the workspace holds per-row partial sums of s^
  //    instead, and one log-sum-exp over J of their column sums serves the row.
  float La[R];
  float Lraw = 0.f;
  const bool raw_sums = d.xa_norm != 0;
  if (__builtin_expect(raw_sums, 0)) {
    float mr = -INFINITY, zr = 0.f;
    for (int J = lane; J < nI; J += 64) {
      float raw = 0.f;
#pragma unroll
      for (int a = 0; a < R; ++a) raw += base[(int64_t)a * nI + J];
      const float x = raw * LOG2E;
      const float mn = fmaxf(mr, x);
      zr = zr * __builtin_amdgcn_exp2f(mr - mn) + __builtin_amdgcn_exp2f(x - mn);
      mr = mn;
    }
    const float mx = wave_max_f32(mr);
    const float z = wave_sum_f32(mr == -INFINITY ? 0.f : zr * __builtin_amdgcn_exp2f(mr - mx));
    Lraw = mx + __builtin_amdgcn_logf(z);
#pragma unroll
    for (int a = 0; a < R; ++a) La[a] = 0.f;
  } else {
    float mr[R], zr[R];
#pragma unroll
    for (int a = 0; a < R; ++a) {
      mr[a] = -INFINITY;
      zr[a] = 0.f;
    }
#pragma unroll 2
    for (int J = lane; J < nI; J += 64) {
      float x[R];
#pragma unroll
      for (int a = 0; a < R; ++a) x[a] = base[(int64_t)a * nI + J];
      // Branch-free update (a divergent branch here made the compiler
      // shuffle all 2R running values on every element).
#pragma unroll
      for (int a = 0; a < R; ++a) {
        const float mn = fmaxf(mr[a], x[a]);
        const float mb = mn == -INFINITY ? 0.f : mn;
        zr[a] = zr[a] * __builtin_amdgcn_exp2f(mr[a] - mb) + __builtin_amdgcn_exp2f(x[a] - mb);
        mr[a] = mn;
      }
    }
#pragma unroll
    for (int a = 0; a < R; ++a) {
      const float mx = wave_max_f32(mr[a]);
      const float z = wave_sum_f32(mr[a] == -INFINITY ? 0.f : zr[a] * __builtin_amdgcn_exp2f(mr[a] - mx));
      La[a] = mx + __builtin_amdgcn_logf(z);
    }
  }
  // 2. Block masses P_J = (1/R) sum_a exp2(lse2[a, J] - La) and integer
  //    weights w = max(1, floor(P * 2^24 + 1/2)).  The masses of a row sum to
  //    1, so every sum of weights below is at most W <= 2^24 (1 + eps) + nI,
  //    exact in 32 bits.
  uint32_t wsum = 0;
  uint32_t wmax = 0;
  float* bm = block_mass ? block_mass + row * d.maxqb : nullptr;
#pragma unroll 2
  for (int J = lane; J < nI; J += 64) {
    float P;
    if (__builtin_expect(raw_sums, 0)) {
      float raw = 0.f;
#pragma unroll
      for (int a = 0; a < R; ++a) raw += base[(int64_t)a * nI + J];
      P = __builtin_amdgcn_exp2f(raw * LOG2E - Lraw);
    } else {
      float acc = 0.f;
#pragma unroll
      for (int a = 0; a < R; ++a) acc += __builtin_amdgcn_exp2f(base[(int64_t)a * nI + J] - La[a]);
      P = acc * (1.0f / R);
    }
    if (bm) bm[J] = P;
    const float x = P * 16777216.0f;
    const float fl = floorf(x);
    uint32_t w = (uint32_t)fl + ((x - fl) >= 0.5f ? 1u : 0u);
    w = w < 1u ? 1u : w;
    wgt[J] = w;
    wsum += w;
    wmax = w > wmax ? w : wmax;
  }
  for (int w = lane; w < d.words; w += 64) bits[w] = 0u;
  const uint64_t W = wave_sum_u32(wsum);
  const uint32_t Wmax = wave_max_u32(wmax);
  const uint64_t tn = (uint64_t)d.tau_num, td = (uint64_t)d.tau_den;
  const uint64_t target = tn * W;
  // 3. v* = largest v with (sum of w_J >= v) * td >= tn * W.
  uint32_t lo = 1, hi = Wmax + 1;
  // Rows of up to 64 * 32 blocks search from registers, NR weights per lane
  // with NR the smallest of 4, 8, 16, 32 that holds the row.
  auto search_regs = [&](auto nr_c) __attribute__((always_inline)) {
    constexpr int NR = decltype(nr_c)::value;
    uint32_t wr[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int J = lane + 64 * k;
      const uint32_t x = wgt[J < nI ? J : 0];
      wr[k] = J < nI ? x : 0u;
    }
    while (hi - lo > 1) {
      const uint32_t mid = lo + (hi - lo) / 2;
      uint32_t sl = 0;
#pragma unroll
      for (int k = 0; k < NR; ++k) sl += wr[k] >= mid ? wr[k] : 0u;
      if ((uint64_t)wave_sum_u32(sl) * td >= target) lo = mid;
      else hi = mid;
    }
  };
  const int nreg = (nI + 63) / 64;
  if (nreg <= 4) {
    search_regs(std::integral_constant<int, 4>());
  } else if (nreg <= 8) {
    search_regs(std::integral_constant<int, 8>());
  } else if (nreg <= 16) {
    search_regs(std::integral_constant<int, 16>());
  } else if (nreg <= 32) {
    search_regs(std::integral_constant<int, 32>());
  } else {
    while (hi - lo > 1) {
      const uint32_t mid = lo + (hi - lo) / 2;
      uint32_t sl = 0;
      for (int J = lane; J < nI; J += 64) sl += wgt[J] >= mid ? wgt[J] : 0u;
      if ((uint64_t)wave_sum_u32(sl) * td >= target) lo = mid;
      else hi = mid;
    }
  }
  const uint32_t vstar = lo;
  uint32_t sg = 0;
  for (int J = lane; J < nI; J += 64) sg += wgt[J] > vstar ? wgt[J] : 0u;
  const uint64_t need = target - (uint64_t)wave_sum_u32(sg) * td;  // > 0 by maximality of v*
  const uint64_t vt = (uint64_t)vstar * td;
  const uint64_t ceq = (need + vt - 1) / vt;  // blocks of weight v* to take, lowest J first
  // 4. Rank of each weight-v* block among equals (J order), then set bits.
  const int chunk = (nI + 63) / 64;
  const int j0 = min(nI, lane * chunk), j1 = min(nI, j0 + chunk);
  uint32_t neq = 0;
  for (int J = j0; J < j1; ++J) neq += wgt[J] == vstar;
  uint64_t rank = wave_inclusive_sum(neq) - neq;
  for (int J = j0; J < j1; ++J) {
    bool sel = wgt[J] > vstar || J == 0 || J == I;
    if (wgt[J] == vstar) {
      sel = sel || rank < ceq;
      ++rank;
    }
    if (sel) atomicOr(&bits[J >> 5], 1u << (J & 31));
  }
  uint32_t cnt = 0;
  for (int w = lane; w < d.words; w += 64) {
    const uint32_t x = bits[w];
    mrow[w] = x;
    cnt += __popc(x);
  }
  const uint64_t count = wave_sum_u32(cnt);
  if (lane == 0) {
    row_count[row] = (int32_t)count;
    const uint64_t pairs = (count - 1) * (uint64_t)(B * B) + (uint64_t)(B * (B + 1) / 2);
    atomicAdd((unsigned long long*)&xa_pairs[(int64_t)b * d.Hq + h], (unsigned long long)pairs);
  }
  if (bm) {
    for (int J = nI + lane; J < d.maxqb; J += 64) bm[J] = 0.f;
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
  const int32_t* pair_bg = (const int32_t*)(w + L.xa_pair_bh);
  const int64_t* pair_items = (const int64_t*)(w + L.xa_pair_items);
  float* lse = (float*)(w + L.xa_lse);
  const dim3 grid((unsigned)device_cus());
#define EA_SCORE(DD, RR, HH, GG)                                                         \
  hipLaunchKernelGGL((k_xa_score<DD, RR, HH, GG>), grid, dim3(XaCfg<DD, RR, HH, GG>::NT), 0, st, d, \
                     q, k, m, pair_bg, pair_items, lse)
#define EA_SCORE_G(DD, RR, HH)                                  \
  do {                                                          \
    if (d.xa_group && (HH) > 1) EA_SCORE(DD, RR, HH, true);     \
    else EA_SCORE(DD, RR, HH, false);                           \
  } while (0)
#define EA_SCORE_H(DD, RR)                          \
  do {                                              \
    if (d.xa_hpi == 4) EA_SCORE_G(DD, RR, 4);       \
    else if (d.xa_hpi == 2) EA_SCORE_G(DD, RR, 2);  \
    else EA_SCORE_G(DD, RR, 1);                     \
  } while (0)
  if (d.D == 128) {
    if (d.r == 4) EA_SCORE_H(128, 4);
    else if (d.r == 8) EA_SCORE_H(128, 8);
    else if (d.r == 16) EA_SCORE_H(128, 16);
    else EA_SCORE_H(128, 32);
  } else {
    if (d.r == 4) EA_SCORE_H(64, 4);
    else if (d.r == 8) EA_SCORE_H(64, 8);
    else if (d.r == 16) EA_SCORE_H(64, 16);
    else EA_SCORE_H(64, 32);
  }
#undef EA_SCORE_H
#undef EA_SCORE_G
#undef EA_SCORE
  return hipGetLastError();
}

hipError_t launch_xa_select(const EaDims& d, const uint8_t* modes, const SeqMeta& m, void* ws,
                            const WsLayout& L, uint32_t* mask, int32_t* row_count, int64_t* xa_pairs,
                            float* block_mass, hipStream_t st) {
  const float* lse = (const float*)((char*)ws + L.xa_lse);
  const size_t per_row = (size_t)(d.maxqb + d.words) * 4;  // LDS per wave (row)
  const int rpw = per_row * 4 <= 40960 ? 4 : per_row * 2 <= 40960 ? 2 : 1;
  const int64_t rows = d.nqb_max * d.Hq;
  const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
  const size_t shm = per_row * rpw;
  if (d.r == 4)
    hipLaunchKernelGGL((k_xa_select<4>), grid, dim3(64 * rpw), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  else if (d.r == 8)
    hipLaunchKernelGGL((k_xa_select<8>), grid, dim3(64 * rpw), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  else if (d.r == 16)
    hipLaunchKernelGGL((k_xa_select<16>), grid, dim3(64 * rpw), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  else
    hipLaunchKernelGGL((k_xa_select<32>), grid, dim3(64 * rpw), shm, st, d, modes, m, lse, mask,
                       row_count, xa_pairs, block_mass);
  return hipGetLastError();
}

}  // namespace ea
