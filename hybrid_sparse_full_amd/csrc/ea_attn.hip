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
// Staging: LDS rings of two K tiles and three V^T tiles (160 KB for
// B = d = 128), filled by global->LDS DMA (global_load_lds_dwordx4) one tile
// ahead; one barrier per tile orders the rings.  The two heads of a group run
// half a tile apart (head 1 applies P V of tile t-1 before S of tile t), so
// on every SIMD the softmax of one wave overlaps the MFMAs of the other.  The DMA is issued from inline
// assembly and its completion is tracked by hand (s_waitcnt vmcnt), because
// the compiler's own tracking of LDS DMA waits for every outstanding load.
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
// Softmax: exp2 with the scale c*log2(e) folded into one FMA; the running max
// is shared by both half-waves; O is rescaled only when some max grows.
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
  static constexpr int KBUF = 2;                   // K tiles resident: t, t+1
  static constexpr int VBUF = HPW == 2 ? 3 : 2;    // V^T tiles: t-1 (lagging head), t, t+1
  static_assert(REGIONS % NW == 0, "DMA regions must split evenly over waves");
};

// 16 bytes per lane from global memory (scalar base + 32-bit per-lane byte
// offset) straight into LDS at m0 + 16 * lane.
__device__ inline void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
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

template <int D, int B, int HPW>
__global__ __launch_bounds__(HPW * (B / 32) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn(EaDims d, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const uint16_t* __restrict__ vt, const uint8_t* __restrict__ modes, SeqMeta m,
            const int32_t* __restrict__ sorted_units, const int64_t* __restrict__ row_off,
            const int32_t* __restrict__ row_cost, const uint32_t* __restrict__ tiles,
            uint16_t* __restrict__ o, float* __restrict__ lse) {
  using C = AttnCfg<D, B, HPW>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(C::KBUF + C::VBUF) * C::TILE_ELEMS];

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
  const int64_t off = row_off[row];
  const int32_t cnt = row_cost[row];

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
  const int64_t vrow0 = (int64_t)g * D * d.tpad;
  const int64_t vkey0 = (int64_t)m.qb_prefix[b] * B;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // Token-mask limits of this lane: key j is allowed iff j <= jmax and
  // (j < jsink or j >= jwin).
  const int32_t jmax = min(qi, len - 1);
  const int32_t jsink = mode == EA_MODE_SSA ? d.sink : 0x3fffffff;
  const int32_t jwin = qi - d.window + 1;

  // LDS: K ring then V^T ring.  DMA region R (1 KB) of a tile holds rows
  // R * RPR .. R * RPR + RPR - 1; lane l writes row R * RPR + l / CH, physical
  // chunk l % CH, which holds logical chunk (l % CH) ^ (row % CH).  Row and
  // chunk offsets split into a lane part (held in three registers) and a
  // uniform part (folded into the scalar base); the swizzle's dependence on R
  // is a uniform XOR.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t krowb = (uint32_t)(d.Hkv * D * 2);  // bytes between K tokens
  const uint32_t vrowb = (uint32_t)(d.tpad * 2);      // bytes between V^T rows
  const uint32_t kc16 = (uint32_t)(((lane % C::KCH) ^ (lane / C::KCH)) * 16);
  const uint32_t klane = (uint32_t)(lane / C::KCH) * krowb;
  const uint32_t vc16 = (uint32_t)(((lane % C::VCH) ^ (lane / C::VCH)) * 16);
  const uint32_t vlane = (uint32_t)(lane / C::VCH) * vrowb;
  auto issue_k = [&](int buf, int32_t J) {
    const uint32_t lbase = lds0 + (uint32_t)buf * C::TILE_BYTES;
    const int64_t ktok0 = tok0 + (int64_t)J * B;
    const char* kb = (const char*)(k + (ktok0 * d.Hkv + g) * D);
    if (ktok0 + B <= (int64_t)d.T) {
      // Rows past the sequence end read the next tokens of the buffer; the
      // tile is flagged and those keys are masked.
#pragma unroll
      for (int i = 0; i < C::NI_K; ++i) {
        const int R = wv * C::NI_K + i;
        const uint32_t xr = C::RPR_K < C::KCH ? (uint32_t)(C::RPR_K * (R % (C::KCH / C::RPR_K)) * 16) : 0u;
        dma16(kb + (size_t)R * C::RPR_K * krowb, klane + (kc16 ^ xr), lds_region(lbase, R));
      }
    } else {
      // Tile reaches past the token buffer: clamp rows to the last token.
#pragma unroll
      for (int i = 0; i < C::NI_K; ++i) {
        const int R = wv * C::NI_K + i;
        const int r = R * C::RPR_K + lane / C::KCH;
        const int rc = (int)min<int64_t>(r, (int64_t)d.T - 1 - ktok0);
        const int c = (lane % C::KCH) ^ (r & (C::KCH - 1));
        dma16(kb, (uint32_t)rc * krowb + (uint32_t)c * 16u, lds_region(lbase, R));
      }
    }
  };
  auto issue_v = [&](int buf, int32_t J) {
    const uint32_t lbase = lds0 + (uint32_t)(C::KBUF + buf) * C::TILE_BYTES;
    const char* vb = (const char*)(vt + vrow0 + vkey0 + (int64_t)J * B);
#pragma unroll
    for (int i = 0; i < C::NI_K; ++i) {
      const int R = wv * C::NI_K + i;
      const uint32_t xr = C::RPR_V < C::VCH ? (uint32_t)(C::RPR_V * (R % (C::VCH / C::RPR_V)) * 16) : 0u;
      dma16(vb + (size_t)R * C::RPR_V * vrowb, vlane + (vc16 ^ xr), lds_region(lbase, R));
    }
  };

  f32x16 sacc[C::NKT];
  bf16x8 pb[C::NKT][2];

  // S^T = K Q^T for the B keys of the tile in K buffer `buf`.  k-step outer,
  // sub-tile inner: consecutive MFMAs use independent accumulators, and the
  // K fragments of the next k-step are read while the current ones multiply.
  auto compute_s = [&](int buf) {
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
    for (int s = 0; s < C::KSTEPS; s += 2) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) fb[kt] = kfrag(kt, s + 1);
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
    }
    // Keep the reads one k-step ahead of the MFMAs that consume them.
    sched_reads_ahead<C::NKT, C::KSTEPS>();
  };

  // Token mask (flagged tiles), online-softmax statistics and P = exp2(.) in bf16.
  auto softmax = [&](uint32_t e) {
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
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    rescale = __any(mnew > mrun);
    alpha = __builtin_amdgcn_exp2f((mrun - mref) * C2);
    mrun = mnew;
    const float mb = mref * C2;
    // Row sum in fp32 (the bf16 copy of P only feeds the PV MFMA; summing the
    // rounded copy would cost the LSE up to 2^-9 relative on short rows).
    float psum = 0.f;
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
    }
    lrun = (rescale ? lrun * alpha : lrun) + psum;
  };

  // O^T += V^T P^T with the V^T tile in buffer `buf` (after the owed rescale).
  auto compute_pv = [&](int buf) {
    if (rescale) {
#pragma unroll
      for (int tt = 0; tt < C::NDT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[tt][r] *= alpha;
    }
    const uint16_t* Vs = smem + (C::KBUF + buf) * C::TILE_ELEMS;
    // k-step (16 keys) outer, d-tile inner: independent accumulators back to
    // back, V^T fragments of the next k-step read ahead.
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
    for (int ks = 0; ks < KS; ks += 2) {
#pragma unroll
      for (int tt = 0; tt < C::NDT; ++tt) fb[tt] = vfrag(tt, ks + 1);
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
    }
    sched_reads_ahead<C::NDT, KS>();
  };

  // Tile loop.  At the top of iteration t every wave waits for its own DMA of
  // tile t and joins the barrier; then K(t+1) and V(t+1) are issued into the
  // ring slots freed by iteration t-1 and stream in while tile t is computed.
  // Head 0 of the group runs S(t) -> softmax(t) -> PV(t); head 1 runs
  // PV(t-1) -> S(t) -> softmax(t), half a tile behind.  Each SIMD holds one
  // wave of each head, so the softmax of one overlaps the MFMAs of the other.
  const bool lag = HPW == 2 && hsub == 1;
  bool pending = false;  // lagging head: P of the previous tile awaits its PV
  int pend_vbuf = 0;
  if (cnt > 0) {
    uint32_t ecur = tiles[off];
    issue_k(0, (int32_t)(ecur & TILE_J_MASK));
    issue_v(0, (int32_t)(ecur & TILE_J_MASK));
    for (int t = 0; t < cnt; ++t) {
      const uint32_t enext = t + 1 < cnt ? tiles[off + t + 1] : 0u;
      wait_vm_barrier<0>();
      if (t + 1 < cnt) {
        issue_k((t + 1) % C::KBUF, (int32_t)(enext & TILE_J_MASK));
        issue_v((t + 1) % C::VBUF, (int32_t)(enext & TILE_J_MASK));
      }
      const bool mine = (ecur & mybit) != 0;
      if (!lag) {
        if (mine) {
          compute_s(t % C::KBUF);
          softmax(ecur);
          compute_pv(t % C::VBUF);
        }
      } else {
        if (pending) compute_pv(pend_vbuf);
        if (mine) {
          compute_s(t % C::KBUF);
          softmax(ecur);
        }
        pending = mine;
        pend_vbuf = t % C::VBUF;
      }
      ecur = enext;
    }
    if (pending) compute_pv(pend_vbuf);
  }

  const float ltot = lrun + __shfl_xor(lrun, 32, 64);
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

hipError_t launch_attention(const EaDims& d, const uint16_t* q, const uint16_t* k,
                            const uint8_t* modes, const SeqMeta& m, void* ws, const WsLayout& L,
                            uint16_t* o, float* lse, hipStream_t st) {
  char* w = (char*)ws;
  const uint16_t* vt = (const uint16_t*)(w + L.vt);
  const int32_t* sorted_units = (const int32_t*)(w + L.sorted_units);
  const int64_t* row_off = (const int64_t*)(w + L.row_off);
  const int32_t* row_cost = (const int32_t*)(w + L.row_cost);
  const uint32_t* tiles = (const uint32_t*)(w + L.tiles);
  const int64_t units = d.nqb_max * d.Hkv;
  const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * d.ngr);
#define EA_ATTN(DD, BB, HH)                                                                     \
  hipLaunchKernelGGL((k_attn<DD, BB, HH>), dim3(grid), dim3(AttnCfg<DD, BB, HH>::NT), 0, st, d, \
                     q, k, vt, modes, m, sorted_units, row_off, row_cost, tiles, o, lse)
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
