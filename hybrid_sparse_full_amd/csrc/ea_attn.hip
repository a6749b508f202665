// Fused hybrid-head flash attention (prefill) for gfx950.
//
// One workgroup per row = (sequence, q-head, q-block of B queries); B / 32
// waves, each owning 32 queries.  The row walks its kv tiles from the flat
// work list, whatever the head's mode (FA, SSA or XA): the mode only decides
// which tiles are listed and, on flagged tiles, the token-level mask.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64):
//   S^T = K Q^T   A = K rows from LDS (key per lane), B = Q in registers
//                 (query per lane), so the accumulator holds one query per
//                 lane and 16 keys per 32-key sub-tile: row statistics of the
//                 online softmax are in-lane plus one exchange between the
//                 two half-waves.
//   O^T += V^T P^T  A = V^T from LDS (d per lane), B = P^T straight from the
//                 S^T accumulator after exp2 and bf16 packing.  The key order
//                 inside each 32-key group of V^T is permuted (bits 2 and 3 of
//                 the key index swapped) when V is transposed, so that the
//                 registers of P^T line up with the MFMA K index without any
//                 data movement.
// Softmax: exp2 with the scale c*log2(e) folded into one FMA; the running max
// is shared by both half-waves; O is rescaled only when some max grows.
#include "ea_device.h"

namespace ea {

template <int D, int B>
struct AttnCfg {
  static constexpr int NW = B / 32;   // waves per workgroup
  static constexpr int NT = NW * 64;  // threads
  static constexpr int KCH = D / 8;   // 16-byte chunks per K row
  static constexpr int VCH = B / 8;   // 16-byte chunks per V^T row
  static constexpr int KSTEPS = D / 16;
  static constexpr int NKT = B / 32;  // 32-key sub-tiles per kv tile
  static constexpr int NDT = D / 32;  // 32-row d tiles of O^T
};

template <int D, int B>
__global__ __launch_bounds__((B / 32) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn(EaDims d, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const uint16_t* __restrict__ vt, const uint8_t* __restrict__ modes, SeqMeta m,
            const int32_t* __restrict__ sorted_units, const int64_t* __restrict__ row_off,
            const int32_t* __restrict__ row_cost, const uint32_t* __restrict__ tiles,
            uint16_t* __restrict__ o, float* __restrict__ lse) {
  using C = AttnCfg<D, B>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[B * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[D * B];

  // XCD-aware decode: blocks b, b+8, b+16, ... run on the same XCD; the G
  // GQA siblings of one unit get consecutive slots there.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int sidx = bid >> 3;
  const int64_t slot = (int64_t)(sidx / d.G) * 8 + xcd;
  const int kq = sidx % d.G;
  if (slot >= m.scal[SCAL_N_UNITS]) return;
  const int32_t u = sorted_units[slot];
  const int64_t row = (int64_t)u * d.G + kq;
  const int32_t qbg = u / d.Hkv;
  const int g = u % d.Hkv;
  const int h = g * d.G + kq;
  const int32_t b = m.qb2seq[qbg];
  const int32_t I = qbg - m.qb_prefix[b];
  const int32_t len = m.len[b];
  const int64_t tok0 = m.start[b];
  const int mode = sane_mode(modes[(int64_t)b * d.Hkv + g]);
  const int64_t off = row_off[row];
  const int32_t cnt = row_cost[row];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int32_t qi = I * B + wave * 32 + l32;  // local query index of this lane
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
  const float C2 = d.scale * LOG2E;
  const int64_t vrow0 = (int64_t)g * D * d.tpad;
  const int64_t vkey0 = (int64_t)m.qb_prefix[b] * B;

  for (int t = 0; t < cnt; ++t) {
    const uint32_t e = tiles[off + t];
    const int32_t J = (int32_t)(e & ~TILE_MASK_FLAG);
    const bool needmask = (e & TILE_MASK_FLAG) != 0;
    __syncthreads();
    {
      const int64_t ktok0 = tok0 + (int64_t)J * B;
      const int32_t kvalid = min(B, len - J * B);
#pragma unroll
      for (int c = tid; c < B * C::KCH; c += C::NT) {
        const int r = c / C::KCH, ch = c % C::KCH;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < kvalid) val = *(const uint4*)(k + ((ktok0 + r) * d.Hkv + g) * D + ch * 8);
        *(uint4*)(Ks + r * D + ((ch ^ (r & (C::KCH - 1))) * 8)) = val;
      }
#pragma unroll
      for (int c = tid; c < D * C::VCH; c += C::NT) {
        const int dd = c / C::VCH, ch = c % C::VCH;
        const uint4 val = *(const uint4*)(vt + vrow0 + (int64_t)dd * d.tpad + vkey0 + (int64_t)J * B + ch * 8);
        *(uint4*)(Vs + dd * B + ((ch ^ (dd & (C::VCH - 1))) * 8)) = val;
      }
    }
    __syncthreads();

    // S^T = K Q^T for the B keys of this tile.
    f32x16 sacc[C::NKT];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
      const int kr = 32 * kt + l32;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const bf16x8 a = *(const bf16x8*)(Ks + kr * D + (((2 * s + half) ^ (kr & (C::KCH - 1))) * 8));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
      }
    }

    if (needmask) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t j = J * B + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          bool ok = (j <= qi) && (j < len);
          if (mode == EA_MODE_SSA) ok = ok && ((j < d.sink) || (qi - j < d.window));
          if (!ok) sacc[kt][r] = -INFINITY;
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
    if (__any(mnew > mrun)) {
      const float alpha = __builtin_amdgcn_exp2f((mrun - mref) * C2);
      lrun *= alpha;
#pragma unroll
      for (int tt = 0; tt < C::NDT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[tt][r] *= alpha;
    }
    mrun = mnew;
    const float mb = mref * C2;

    bf16x8 pb[C::NKT][2];
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
    lrun += psum;

    // O^T += V^T P^T
#pragma unroll
    for (int tt = 0; tt < C::NDT; ++tt) {
      const int dr = 32 * tt + l32;
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int ch = 4 * kt + 2 * mm + half;
          const bf16x8 a = *(const bf16x8*)(Vs + dr * B + ((ch ^ (dr & (C::VCH - 1))) * 8));
          oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][mm], oacc[tt], 0, 0, 0);
        }
    }
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
      lse[(int64_t)h * d.T + tok0 + qi] = ltot > 0.f ? (mrun * d.scale + log2f(ltot) * LN2) : -INFINITY;
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
  const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * d.G);
#define EA_ATTN(DD, BB)                                                                          \
  hipLaunchKernelGGL((k_attn<DD, BB>), dim3(grid), dim3(AttnCfg<DD, BB>::NT), 0, st, d, q, k, vt, \
                     modes, m, sorted_units, row_off, row_cost, tiles, o, lse)
  if (d.D == 128 && d.B == 128) EA_ATTN(128, 128);
  else if (d.D == 128 && d.B == 64) EA_ATTN(128, 64);
  else if (d.D == 64 && d.B == 128) EA_ATTN(64, 128);
  else EA_ATTN(64, 64);
#undef EA_ATTN
  return hipGetLastError();
}

}  // namespace ea
