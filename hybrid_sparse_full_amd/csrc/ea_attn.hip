// Fused hybrid-head flash attention (prefill) for gfx950.
//
// One workgroup per row of the work list = (sequence, q-block of B queries,
// group of HPW GQA sibling q-heads of one KV head).  Each head uses B / 32
// waves of 32 queries; the heads of a group share every K / V tile staged in
// LDS.  The row walks its kv tiles from the flat work list whatever the
// mode (FA, SSA or XA): the mode only decided which tiles were listed and,
// on flagged tiles, the token-level mask.  XA heads of one group may select
// different blocks; the list holds their union and a wave skips the tiles
// that its head does not attend.
//
// Staging: LDS rings of two K tiles and two V^T tiles (128 KB for
// B = d = 128), filled by global->LDS DMA (global_load_lds_dwordx4) one
// period ahead; one barrier per tile orders the rings.  Every wave runs
// PV(t-1) and S(t) on the matrix core and the softmax of tile t on the
// vector ALU; the two heads of a group do so half a period apart, so on
// every SIMD the softmax of one wave overlaps the MFMAs of the other.  The
// DMA is issued from inline assembly and its completion is tracked by hand
// (s_waitcnt vmcnt), because the compiler's own tracking of LDS DMA waits
// for every outstanding load.  For the same reason the work-list entries
// reach the waves through LDS too: wave 0 copies entry n into a four-slot
// ring by DMA three periods ahead, and every wave reads it one period ahead,
// so no global load (and no compiler-inserted vmcnt wait) sits in the loop.
// The LDS image of each tile row is XOR-swizzled in 16-byte chunks so that
// the MFMA operand reads are free of bank conflicts.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T = K Q^T   A = K rows from LDS (key per lane), B = Q in registers
//                 (query per lane): the accumulator holds one query per lane
//                 and 16 keys per 32-key sub-tile, so the online-softmax row
//                 statistics are in-lane plus one exchange between the two
//                 half-waves.
//   O^T += V^T P^T  A = V^T from LDS (d per lane), B = P^T straight from the
//                 S^T accumulator after exp2 and bf16 packing.  The key order
//                 inside each 32-key group of V^T is permuted (bits 2 and 3 of
//                 the key index swapped) when V is transposed, so the registers
//                 of P^T line up with the MFMA K index with no data movement.
// Softmax: exp2 with the scale c*log2(e) folded into one FMA against a lazy
// reference max, shared by both half-waves (v_permlane32_swap, no LDS).
// Once every row of the wave has a finite reference, a tile's row maxima are
// not formed at all: P is computed straight away and each lane's sum of its
// P values, which bounds every one of them, decides whether the tile must be
// redone on the exact path.  That path forms the row maxima and moves the
// reference only when a row max exceeds it by more than 2^8 in the exp2
// domain, so O and l are rescaled rarely.  P stays at most 2^14, far inside
// the range of bf16 and fp32, and keeps their relative precision.
#include "ea_device.h"

namespace ea {

template <int D, int B, int HPW>
struct AttnCfg {
  static constexpr int WPH = B / 32;               // waves per head
  static constexpr int NW = HPW * WPH;             // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int KCH = D / 8;                // 16-byte chunks per K row
  static constexpr int VCH = B / 8;                // 16-byte chunks per V^T row
  static constexpr int TILE_ELEMS = B * D;
  static constexpr int TILE_BYTES = TILE_ELEMS * 2;
  static constexpr int REGIONS = TILE_BYTES / 1024; // 1 KB DMA regions per tile
  static constexpr int NI_K = REGIONS / NW;        // DMA instructions per wave per tile
  static constexpr int NI = 2 * NI_K;              // per stage (K and V^T)
  static constexpr int RPR_K = 1024 / (D * 2);     // K rows per region
  static constexpr int RPR_V = 1024 / (B * 2);     // V^T rows per region
  static constexpr int KSTEPS = D / 16;
  static constexpr int NKT = B / 32;               // 32-key sub-tiles per kv tile
  static constexpr int NDT = D / 32;               // 32-row d tiles of O^T
  static constexpr int KBUF = 2;                   // K tiles resident: t (in use), t+1 (landing)
  static constexpr int VBUF = 2;                   // V^T tiles: t-1 (in use), t (landing)
  static_assert(REGIONS % NW == 0, "DMA regions must split evenly over waves");
};

// 16 bytes per lane from global memory (scalar base + 32-bit per-lane byte
// offset) straight into LDS at m0 + 16 * lane.  No "memory" clobber: the LDS
// slot written here is read only after the next workgroup barrier (whose asm
// does carry one), so the scheduler may move LDS reads and MFMAs across it.
__device__ inline void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // The base is wave-uniform by construction; readfirstlane states it.
  // (readfirstlane returns int: widen through uint32_t, never sign-extend.)
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"((const void*)(uintptr_t)bs), "s"(lds_addr)
               : "m0");
}

// Scheduling pattern for an LDS-fed MFMA sequence of STEPS k-steps with N
// independent accumulators: fragment reads run two k-steps ahead of the
// MFMAs that consume them.
template <int N, int STEPS>
__device__ inline void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * N, 0);
#pragma unroll
  for (int i = 0; i < STEPS - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, N, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, N, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * N, 0);
}

__device__ inline uint32_t lds_region(uint32_t base, int R) {
  return __builtin_amdgcn_readfirstlane(base + (uint32_t)R * 1024u);
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then join the workgroup barrier.
template <int N>
__device__ inline void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// 4 bytes from global memory (scalar address) into LDS at m0, issued by the
// active lanes (one, at the call site).
__device__ inline void dma4(const void* sbase, uint32_t lds_addr) {
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(0u), "s"((const void*)(uintptr_t)bs), "s"(lds_addr)
               : "m0");
}

template <int D, int B, int HPW>
__global__ __launch_bounds__(HPW * (B / 32) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn(EaDims d, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
            const uint16_t* __restrict__ vp, const uint8_t* __restrict__ modes, SeqMeta m,
            const int32_t* __restrict__ sorted_units, const int64_t* __restrict__ row_off,
            const int32_t* __restrict__ row_cost, const uint32_t* __restrict__ tiles,
            uint16_t* __restrict__ o, float* __restrict__ lse) {
  using C = AttnCfg<D, B, HPW>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(C::KBUF + C::VBUF) * C::TILE_ELEMS];
  // Ring of four list entries: entry n is copied into slot n & 3 by wave 0
  // three periods ahead of its use and read by every wave one period ahead.
  __shared__ uint32_t elist[4];

  // XCD-aware decode: blocks b, b+8, b+16, ... run on the same XCD; the head
  // groups of one unit (q-block, KV head) get consecutive slots there.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int sidx = bid >> 3;
  const int64_t slot = (int64_t)(sidx / d.ngr) * 8 + xcd;
  const int kg = sidx % d.ngr;
  if (slot >= m.scal[SCAL_N_UNITS]) return;
  const int32_t u = sorted_units[slot];
  const int64_t row = (int64_t)u * d.ngr + kg;
  const int32_t qbg = u / d.Hkv;
  const int g = u % d.Hkv;
  const int32_t b = m.qb2seq[qbg];
  const int32_t I = qbg - m.qb_prefix[b];
  const int32_t len = m.len[b];
  const int64_t tok0 = m.start[b];
  const int mode = sane_mode(modes[(int64_t)b * d.Hkv + g]);
  // Row data is wave-uniform: keep it (and so every DMA address) in SGPRs.
  const int64_t off = uniform64(row_off[row]);
  const int32_t cnt = __builtin_amdgcn_readfirstlane(row_cost[row]);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int hsub = wave / C::WPH;  // head within the group
  const int wq = wave % C::WPH;
  const int h = g * d.G + kg * HPW + hsub;
  const uint32_t mybit = TILE_HEAD0 << hsub;
  const int32_t qi = I * B + wq * 32 + l32;  // local query index of this lane
  const bool qvalid = qi < len;

  bf16x8 qf[C::KSTEPS];
  {
    const uint16_t* qrow = q + ((tok0 + (qvalid ? qi : 0)) * d.Hq + h) * D;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qvalid) v = *(const uint4*)(qrow + 16 * s + 8 * half);
      qf[s] = *(const bf16x8*)&v;
    }
  }

  f32x16 oacc[C::NDT];
#pragma unroll
  for (int t = 0; t < C::NDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  float alpha = 1.f;       // rescale of O still owed before the next PV
  bool rescale = false;
  const float C2 = d.scale * LOG2E;
  // Packed tiles of this KV head: tile of kv block J at (g * nqb_max + P_b + J).
  const int64_t tile0 = uniform64((int64_t)g * d.nqb_max + m.qb_prefix[b]);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // Token-mask limits of this lane: key j is allowed iff j <= jmax and
  // (j < jsink or j >= jwin).
  const int32_t jmax = min(qi, len - 1);
  const int32_t jsink = mode == EA_MODE_SSA ? d.sink : 0x3fffffff;
  const int32_t jwin = qi - d.window + 1;

  // LDS: K ring then V^T ring.  Packed tiles are contiguous and zero padded.
  // DMA region R (1 KB) of a tile holds rows R * RPR .. R * RPR + RPR - 1;
  // lane l writes row R * RPR + l / CH, physical chunk l % CH, which must
  // hold logical chunk (l % CH) ^ (row % CH).  The byte offset in the tile is
  // R * 1024 (uniform, into the scalar base) + (lk ^ xr(R)) with a lane
  // constant lk and a uniform XOR xr(R).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lk = (uint32_t)((lane / C::KCH) * (D * 2) + 16 * ((lane % C::KCH) ^ (lane / C::KCH)));
  const uint32_t lv = (uint32_t)((lane / C::VCH) * (B * 2) + 16 * ((lane % C::VCH) ^ (lane / C::VCH)));
  // DMA instruction i (0 <= i < NI_K) of this wave for the K tile of block
  // J into K ring slot `buf` (resp. the V^T tile into V ring slot `buf`).
  auto dma_k = [&](int buf, int32_t J, int i) {
    const int R = wv * C::NI_K + i;
    const uint32_t xr = C::RPR_K < C::KCH ? (uint32_t)(C::RPR_K * (R % (C::KCH / C::RPR_K)) * 16) : 0u;
    const char* src = (const char*)(kp + (tile0 + J) * C::TILE_ELEMS) + R * 1024;
    dma16(src, lk ^ xr, lds_region(lds0 + (uint32_t)buf * C::TILE_BYTES, R));
  };
  auto dma_v = [&](int buf, int32_t J, int i) {
    const int R = wv * C::NI_K + i;
    const uint32_t xr = C::RPR_V < C::VCH ? (uint32_t)(C::RPR_V * (R % (C::VCH / C::RPR_V)) * 16) : 0u;
    const char* src = (const char*)(vp + (tile0 + J) * C::TILE_ELEMS) + R * 1024;
    dma16(src, lv ^ xr, lds_region(lds0 + (uint32_t)(C::KBUF + buf) * C::TILE_BYTES, R));
  };

  // DMA of one period: this wave's NI_K instructions for the K tile of
  // block jk (ring slot nk) and its NI_K for the V^T tile of block jv (ring
  // slot nv); a block of -1 means nothing to load.  The softmax phase of n
  // sub-tiles issues, at sub-tile j, the instructions with index in
  // [j * per, (j + 1) * per), per = ceil(NI_K / n), so their issue overlaps
  // the exponentials.
  int32_t jk = -1, jv = -1;
  int nk = 0, nv = 0;
  auto dma_k_part = [&](int j, int n) {
    const int per = (C::NI_K + n - 1) / n;
#pragma unroll
    for (int x = 0; x < per; ++x) {
      const int idx = j * per + x;
      if (idx < C::NI_K && __builtin_expect(jk >= 0, 1)) dma_k(nk, jk, idx);
    }
  };
  auto dma_v_part = [&](int j, int n) {
    const int per = (C::NI_K + n - 1) / n;
#pragma unroll
    for (int x = 0; x < per; ++x) {
      const int idx = j * per + x;
      if (idx < C::NI_K && __builtin_expect(jv >= 0, 1)) dma_v(nv, jv, idx);
    }
  };

  f32x16 sacc[C::NKT];
  bf16x8 pb[C::NKT][2];

  // S^T = K Q^T for the B keys of the tile in K buffer `buf`.  k-step outer,
  // sub-tile inner: consecutive MFMAs use independent accumulators and the K
  // fragments are read two k-steps ahead (the order is pinned for the
  // scheduler).  With `dma`, this wave's share of the period's V^T DMA is
  // issued right after the first fragment reads, so its issue overlaps their
  // latency.
  auto compute_s = [&](int buf, bool dma) __attribute__((always_inline)) {
    const uint16_t* Ks = smem + buf * C::TILE_ELEMS;
    auto kfrag = [&](int kt, int s) {
      const int kr = 32 * kt + l32;
      return *(const bf16x8*)(Ks + kr * D + (((2 * s + half) ^ (kr & (C::KCH - 1))) * 8));
    };
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
    bf16x8 fa[C::NKT], fb[C::NKT];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) fa[kt] = kfrag(kt, 0);
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) fb[kt] = kfrag(kt, 1);
    if (dma && __builtin_expect(jv >= 0, 1)) {
#pragma unroll
      for (int i = 0; i < C::NI_K; ++i) dma_v(nv, jv, i);
    }
#pragma unroll
    for (int s = 0; s < C::KSTEPS; s += 2) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kt], qf[s], sacc[kt], 0, 0, 0);
      if (s + 2 < C::KSTEPS) {
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) fa[kt] = kfrag(kt, s + 2);
      }
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kt], qf[s + 1], sacc[kt], 0, 0, 0);
      if (s + 3 < C::KSTEPS) {
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) fb[kt] = kfrag(kt, s + 3);
      }
    }
    sched_reads_ahead<C::NKT, C::KSTEPS>();
  };

  // Token mask (flagged tiles), online-softmax statistics and P = exp2(.) in
  // bf16.  With `dma`, this wave's whole DMA share of the period is issued
  // between the exponentials of the NKT sub-tiles.
  auto softmax = [&](uint32_t e, bool dma) __attribute__((always_inline)) {
    if (__builtin_expect((e & TILE_MASK_FLAG) != 0, 0)) {
      // A real branch: only flagged tiles pay for the token mask.
      asm volatile("");
      const int32_t jb = (int32_t)(e & TILE_J_MASK) * B + 4 * half;
      const int32_t hi_rel = jmax - jb, sink_rel = jsink - jb, win_rel = jwin - jb;
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t c = 32 * kt + 8 * (r >> 2) + (r & 3);
          const bool ok = (c <= hi_rel) & ((c < sink_rel) | (c >= win_rel));
          sacc[kt][r] = ok ? sacc[kt][r] : -INFINITY;
        }
    }
    // P = exp2(c s - c m) in fp32, its lane sum, and the bf16 copy for the PV
    // MFMA (the row sum stays in fp32: summing the rounded copy would cost the
    // LSE up to 2^-9 relative on short rows).
    float psum = 0.f;
    auto exps = [&](float mb, bool issue) __attribute__((always_inline)) {
      psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
        f32x8 p0, p1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          p0[r] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], C2, -mb));
          p1[r] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 + r], C2, -mb));
          psum += p0[r] + p1[r];
        }
        pb[kt][0] = __builtin_convertvector(p0, bf16x8);
        pb[kt][1] = __builtin_convertvector(p1, bf16x8);
        if (issue) {
          dma_k_part(kt, C::NKT);
          dma_v_part(kt, C::NKT);
        }
      }
    };
    // Fast path: every row of the wave has a finite reference max mrun.  A
    // lane sum above 2^14 means some P exceeded 2^8, i.e. a row max rose by
    // more than 2^8 in the exp2 domain: the wave redoes the tile below.  The
    // sum is +inf, never NaN, if an exponential overflows.
    rescale = false;
    const bool cold = __any(mrun == -INFINITY);
    if (__builtin_expect(!cold, 1)) exps(mrun * C2, dma);
    if (__builtin_expect(cold || __any(psum > 16384.f), 0)) {
      // Exact path: row maxima of the tile; the reference max moves only when
      // one exceeds it by more than 2^8 in the exp2 domain (or is its first
      // finite value).  l and O always refer to the same mrun.
      asm volatile("");
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
      mx = halves_max(mx);
      rescale = __any((mx - mrun) * C2 > 8.0f);
      if (rescale) {
        const float mnew = fmaxf(mrun, mx);
        alpha = __builtin_amdgcn_exp2f((mrun - ((mnew == -INFINITY) ? 0.f : mnew)) * C2);
        mrun = mnew;
      }
      // The DMA share went out with the fast path unless it was skipped.
      exps(((mrun == -INFINITY) ? 0.f : mrun) * C2, dma && cold);
    }
    lrun = (rescale ? lrun * alpha : lrun) + psum;
  };

  // O^T += V^T P^T with the V^T tile in buffer `buf` (after the owed
  // rescale); k-step (16 keys) outer, d-tile inner, V^T fragments two k-steps
  // ahead (order pinned); with `dma`, this wave's share of the period's K
  // DMA is issued right after the first fragment reads.
  auto compute_pv = [&](int buf, bool dma) __attribute__((always_inline)) {
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int tt = 0; tt < C::NDT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[tt][r] *= alpha;
    }
    const uint16_t* Vs = smem + (C::KBUF + buf) * C::TILE_ELEMS;
    auto vfrag = [&](int tt, int ks) {
      const int dr = 32 * tt + l32;
      const int ch = 2 * ks + half;  // = 4 kt + 2 mm + half with ks = 2 kt + mm
      return *(const bf16x8*)(Vs + dr * B + ((ch ^ (dr & (C::VCH - 1))) * 8));
    };
    constexpr int KS = 2 * C::NKT;
    bf16x8 fa[C::NDT], fb[C::NDT];
#pragma unroll
    for (int tt = 0; tt < C::NDT; ++tt) fa[tt] = vfrag(tt, 0);
#pragma unroll
    for (int tt = 0; tt < C::NDT; ++tt) fb[tt] = vfrag(tt, 1);
    if (dma && __builtin_expect(jk >= 0, 1)) {
#pragma unroll
      for (int i = 0; i < C::NI_K; ++i) dma_k(nk, jk, i);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
#pragma unroll
      for (int tt = 0; tt < C::NDT; ++tt)
        oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tt], pb[ks >> 1][ks & 1], oacc[tt], 0, 0, 0);
      if (ks + 2 < KS) {
#pragma unroll
        for (int tt = 0; tt < C::NDT; ++tt) fa[tt] = vfrag(tt, ks + 2);
      }
#pragma unroll
      for (int tt = 0; tt < C::NDT; ++tt)
        oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tt], pb[(ks + 1) >> 1][(ks + 1) & 1], oacc[tt], 0, 0, 0);
      if (ks + 3 < KS) {
#pragma unroll
        for (int tt = 0; tt < C::NDT; ++tt) fb[tt] = vfrag(tt, ks + 3);
      }
    }
    sched_reads_ahead<C::NDT, KS>();
  };

  // Tile loop: one period per tile plus one to drain.  At the top of period
  // t every wave waits for its own DMA and joins the barrier; then K(t) and
  // V^T(t-1) are resident, and the DMA of K(t+1) and V^T(t) goes into the
  // ring slots that period t-1 finished reading.  Every wave runs
  // PV(t-1) -> S(t) on the matrix core and softmax(t) on the vector ALU;
  // head 0 of the group does so in that order, head 1 rotated by half a
  // period: softmax(t-1) -> PV(t-1) -> S(t), holding S(t-1) across the
  // barrier.  On each SIMD (one wave of each head) the exponentials of one
  // wave then run while the other wave's MFMAs do, and the matrix core sees
  // 2 x (PV + S) per period.
  // The two orders are separate loops (chosen once per wave), so that each
  // keeps only its own state live across the barrier: P of the previous
  // tile for head 0, S of the previous tile for head 1.
  auto tile_loop = [&](auto lag_c) __attribute__((always_inline)) {
    constexpr bool LAG = decltype(lag_c)::value;
    bool pend = false;   // the previous tile still owes this wave its PV (LAG: softmax and PV)
    uint32_t epend = 0;  // that tile's list entry
    uint32_t ecur = (uint32_t)__builtin_amdgcn_readfirstlane((int)tiles[off]);
    uint32_t enext = cnt > 1 ? (uint32_t)__builtin_amdgcn_readfirstlane((int)tiles[off + 1]) : 0u;
    const uint32_t elds = (uint32_t)(uintptr_t)elist;
    auto dma_entry = [&](int n) {
      if (wv == 0 && n < cnt && lane == 0) dma4(tiles + off + n, elds + 4u * (uint32_t)(n & 3));
    };
    dma_entry(2);
    jk = (int32_t)(ecur & TILE_J_MASK);
    nk = 0;
#pragma unroll
    for (int i = 0; i < C::NI_K; ++i) dma_k(0, jk, i);
    for (int t = 0; t <= cnt; ++t) {
      wait_vm_barrier<0>();
      // Entry t + 2 landed with the DMA waited for above; entry t + 3 goes out now.
      const uint32_t eraw = elist[(t + 2) & 3];
      dma_entry(t + 3);
      jk = t + 1 < cnt ? (int32_t)(enext & TILE_J_MASK) : -1;
      jv = t < cnt ? (int32_t)(ecur & TILE_J_MASK) : -1;
      nk = (t + 1) & 1;
      nv = t & 1;
      const bool mine = t < cnt && (ecur & mybit) != 0;
      bool kd = false, vd = false;  // this period's K / V^T DMA issued
      // A wave issues its MFMA phase at raised priority, so the other wave's
      // exponentials on the same SIMD fill the gaps between MFMA issues
      // instead of delaying them (measured: 2 % shorter launches; raising the
      // softmax instead made them 1.5 % longer).
      if (!LAG) {
        __builtin_amdgcn_s_setprio(1);
        if (__builtin_expect(pend, 1)) {
          compute_pv((t - 1) & 1, true);
          kd = true;
        }
        if (__builtin_expect(mine, 1)) {
          compute_s(t & 1, true);
          vd = true;
          __builtin_amdgcn_s_setprio(0);
          softmax(ecur, false);
        }
        __builtin_amdgcn_s_setprio(0);
      } else {
        if (__builtin_expect(pend, 1)) {
          softmax(epend, true);
          kd = vd = true;
          __builtin_amdgcn_s_setprio(1);
          compute_pv((t - 1) & 1, false);
        }
        if (__builtin_expect(mine, 1)) {
          __builtin_amdgcn_s_setprio(1);
          compute_s(t & 1, false);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      if (__builtin_expect(!kd, 0)) {
#pragma unroll
        for (int i = 0; i < C::NI_K; ++i)
          if (jk >= 0) dma_k(nk, jk, i);
      }
      if (__builtin_expect(!vd, 0)) {
#pragma unroll
        for (int i = 0; i < C::NI_K; ++i)
          if (jv >= 0) dma_v(nv, jv, i);
      }
      pend = mine;
      epend = ecur;
      ecur = enext;
      enext = t + 2 < cnt ? (uint32_t)__builtin_amdgcn_readfirstlane((int)eraw) : 0u;
    }
  };
  if (cnt > 0) {
    if (HPW == 2 && hsub == 1) tile_loop(std::true_type());
    else tile_loop(std::false_type());
  }

  const float ltot = halves_sum(lrun);
  if (qvalid) {
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    uint16_t* orow = o + ((tok0 + qi) * d.Hq + h) * D;
#pragma unroll
    for (int tt = 0; tt < C::NDT; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[tt][4 * jj + e] * inv;
        const bf16x4 hv = __builtin_convertvector(v, bf16x4);
        *(bf16x4*)(orow + 32 * tt + 8 * jj + 4 * half) = hv;
      }
    if (half == 0)
      lse[(int64_t)h * d.T + tok0 + qi] =
          ltot > 0.f ? (mrun * d.scale + log2f(ltot) * LN2) : -INFINITY;
  }
}

hipError_t launch_attention(const EaDims& d, const uint16_t* q, const uint8_t* modes,
                            const SeqMeta& m, void* ws, const WsLayout& L, uint16_t* o, float* lse,
                            hipStream_t st) {
  char* w = (char*)ws;
  const uint16_t* kp = (const uint16_t*)(w + L.kvp);
  const uint16_t* vp = kp + (size_t)d.Hkv * d.D * (size_t)d.tpad;
  const int32_t* sorted_units = (const int32_t*)(w + L.sorted_units);
  const int64_t* row_off = (const int64_t*)(w + L.row_off);
  const int32_t* row_cost = (const int32_t*)(w + L.row_cost);
  const uint32_t* tiles = (const uint32_t*)(w + L.tiles);
  const int64_t units = d.nqb_max * d.Hkv;
  const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * d.ngr);
#define EA_ATTN(DD, BB, HH)                                                                     \
  hipLaunchKernelGGL((k_attn<DD, BB, HH>), dim3(grid), dim3(AttnCfg<DD, BB, HH>::NT), 0, st, d, \
                     q, kp, vp, modes, m, sorted_units, row_off, row_cost, tiles, o, lse)
  if (d.hpw == 2) {
    if (d.D == 128 && d.B == 128) EA_ATTN(128, 128, 2);
    else if (d.D == 128 && d.B == 64) EA_ATTN(128, 64, 2);
    else if (d.D == 64 && d.B == 128) EA_ATTN(64, 128, 2);
    else EA_ATTN(64, 64, 2);
  } else {
    if (d.D == 128 && d.B == 128) EA_ATTN(128, 128, 1);
    else if (d.D == 128 && d.B == 64) EA_ATTN(128, 64, 1);
    else if (d.D == 64 && d.B == 128) EA_ATTN(64, 128, 1);
    else EA_ATTN(64, 64, 1);
  }
#undef EA_ATTN
  return hipGetLastError();
}

}  // namespace ea
