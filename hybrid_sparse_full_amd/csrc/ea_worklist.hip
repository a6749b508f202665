// Work-list builder of the fused prefill: one flat list of kv tiles for
// every (q-block, q-head) row of every mode, plus a longest-first schedule.
//
//   k_pack   K and V -> contiguous zero-padded tiles per (KV head, q-block):
//            K key-major, V transposed (V^T) with keys permuted inside each
//            32-key group to match the MFMA operand order of the attention
//            kernel.
//   k_cost   tiles per row (FA: I+1, SSA: sink + window blocks, XA: popcount
//            of the union of the group's mask rows); a row is a (q-block,
//            group of 1 or 2 GQA sibling q-heads) that one workgroup serves;
//            per unit (q-block, KV head) the max over its rows; histogram.
//   k_sched  one workgroup: counting sort of units by cost, descending, and
//            the exclusive scan of row costs (row offsets into the list).
//   k_fill   one wave per row writes its kv-block indices, each flagged when
//            the tile needs a token-level mask (diagonal, window edge, sink
//            edge, ragged sequence end).
#include "ea_device.h"

namespace ea {

struct RowInfo {
  int32_t b, I, len, mode;
};

__device__ inline RowInfo decode_qb(const EaDims& d, const SeqMeta& m, int32_t qbg, int g,
                                    const uint8_t* modes, const uint32_t* xa_mask) {
  RowInfo r;
  r.b = m.qb2seq[qbg];
  r.I = qbg - m.qb_prefix[r.b];
  r.len = m.len[r.b];
  r.mode = sane_mode(modes[(int64_t)r.b * d.Hkv + g]);
  if (r.mode == EA_MODE_XA && xa_mask == nullptr) r.mode = EA_MODE_FA;
  return r;
}

// First window block and number of sink-only blocks of an SSA row.
__device__ inline void ssa_ranges(const EaDims& d, int32_t I, int32_t* jlo, int32_t* ns) {
  const int64_t first = (int64_t)I * d.B - d.window + 1;  // window start of the first query
  const int32_t lo = first <= 0 ? 0 : (int32_t)(first / d.B);
  *jlo = lo;
  *ns = min(cdiv(d.sink, d.B), lo);
}

// Does tile (I, J) of a row need a token-level mask?
__device__ inline bool tile_needs_mask(const EaDims& d, int mode, int32_t I, int32_t J,
                                       int32_t len) {
  const int64_t i0 = (int64_t)I * d.B;
  const int64_t ilast = min<int64_t>(i0 + d.B - 1, len - 1);
  const int64_t j0 = (int64_t)J * d.B, j1 = j0 + d.B - 1;
  if (J >= I) return true;               // diagonal (J > I never listed)
  if (j1 >= len) return true;            // keys past the sequence end
  if (mode == EA_MODE_SSA) {
    // Keys before jm are sink keys; every key from jm on is kept for every
    // query of the block iff the last query still has jm inside its window.
    const int64_t jm = max<int64_t>(j0, d.sink);
    if (jm > j1) return false;
    return ilast - jm >= d.window;
  }
  return false;
}

__device__ inline int swap_bits23(int p) {
  return (p & ~0xC) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// ---------------------------------------------------------------- k_pack
// Packs the K and V tiles of every (KV head g, global q-block qbg) into
// contiguous, zero-padded B x d blocks: Kp[g][qbg] = K rows (key-major) and
// Vp[g][qbg] = V^T (d-major, keys permuted inside each 32-key group).
template <int D, int B>
__global__ __launch_bounds__(256) void k_pack(EaDims d, const uint16_t* __restrict__ k,
                                              const uint16_t* __restrict__ v, SeqMeta m,
                                              uint16_t* __restrict__ kp, uint16_t* __restrict__ vp) {
  __shared__ uint16_t tile[B][D + 2];
  const int32_t qbg = blockIdx.x;
  if (qbg >= m.scal[SCAL_TOTAL_QB]) return;
  const int g = blockIdx.y;
  const int32_t b = m.qb2seq[qbg];
  const int32_t J = qbg - m.qb_prefix[b];
  const int32_t len = m.len[b];
  const int64_t tok0 = (int64_t)m.start[b] + (int64_t)J * B;
  const int32_t nvalid = min(B, len - J * B);
  const int64_t tile_off = ((int64_t)g * d.nqb_max + qbg) * (B * D);
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < B * CPR; c += 256) {
    const int key = c / CPR, ch = c % CPR;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (key < nvalid) {
      const int64_t src = ((tok0 + key) * d.Hkv + g) * D + ch * 8;
      kv = *(const uint4*)(k + src);
      vv = *(const uint4*)(v + src);
    }
    *(uint4*)(kp + tile_off + key * D + ch * 8) = kv;
    const uint16_t* pv = (const uint16_t*)&vv;
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[key][ch * 8 + e] = pv[e];
  }
  __syncthreads();
  // V^T rows: 8 consecutive (permuted) key positions per thread.
  constexpr int CPD = B / 8;
  for (int c = threadIdx.x; c < D * CPD; c += 256) {
    const int dd = c / CPD, p0 = (c % CPD) * 8;
    uint16_t outv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = p0 + e;
      const int key = (p & ~31) | swap_bits23(p & 31);
      outv[e] = tile[key][dd];
    }
    *(uint4*)(vp + tile_off + dd * B + p0) = *(const uint4*)outv;
  }
}

// ---------------------------------------------------------------- k_cost
__global__ __launch_bounds__(256) void k_cost(EaDims d, const uint8_t* __restrict__ modes,
                                              const uint32_t* __restrict__ xa_mask, SeqMeta m,
                                              int32_t* __restrict__ unit_cost,
                                              int32_t* __restrict__ row_cost,
                                              int32_t* __restrict__ hist) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = u < m.scal[SCAL_N_UNITS];
  const int32_t qbg = valid ? (int32_t)(u / d.Hkv) : 0;
  const int g = (int)(u % d.Hkv);
  RowInfo ri = {0, 0, 0, EA_MODE_FA};
  if (valid) ri = decode_qb(d, m, qbg, g, modes, xa_mask);
  int32_t uc = 0;
  int64_t head_tiles = 0;
  for (int kg = 0; valid && kg < d.ngr; ++kg) {
    int32_t c;
    if (ri.mode == EA_MODE_SSA) {
      int32_t jlo, ns;
      ssa_ranges(d, ri.I, &jlo, &ns);
      c = ns + ri.I - jlo + 1;
      head_tiles += (int64_t)c * d.hpw;
    } else if (ri.mode == EA_MODE_XA) {
      // Union of the blocks selected by the heads of this group.
      const uint32_t* row = xa_mask + ((int64_t)qbg * d.Hq + g * d.G + kg * d.hpw) * d.words;
      // Words 0 .. I / 32 hold the blocks J <= I; 8 words of both heads
      // (hpw <= 2) are loaded before any is used.
      c = 0;
      const int nw = ri.I / 32 + 1;
      const uint32_t* row1 = row + (d.hpw > 1 ? d.words : 0);
      for (int w0 = 0; w0 < nw; w0 += 8) {
        uint32_t b0[8], b1[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bool in = w0 + t < nw;
          b0[t] = in ? row[w0 + t] : 0u;
          b1[t] = in && d.hpw > 1 ? row1[w0 + t] : 0u;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int hi = ri.I - (w0 + t) * 32;  // keep J <= I
          const uint32_t keep = hi < 0 ? 0u : hi < 31 ? (2u << hi) - 1u : 0xffffffffu;
          const uint32_t a0 = b0[t] & keep, a1 = b1[t] & keep;
          head_tiles += __popc(a0) + __popc(a1);
          c += __popc(a0 | a1);
        }
      }
    } else {
      c = ri.I + 1;
      head_tiles += (int64_t)c * d.hpw;
    }
    row_cost[u * d.ngr + kg] = c;
    uc = max(uc, c);
  }
  // One counter update per wave, and one histogram update per distinct cost
  // in the wave (units of equal cost are common: every SSA row of a head).
  const uint64_t ht = wave_sum((uint64_t)head_tiles);
  if ((threadIdx.x & 63) == 0 && ht) atomicAdd((unsigned long long*)(m.scal + SCAL_HEAD_TILES64), ht);
  if (!valid) return;
  unit_cost[u] = uc;
  uint64_t todo = __ballot(1);
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int32_t c = __shfl(uc, leader, 64);
    const uint64_t same = __ballot(uc == c) & todo;
    if ((threadIdx.x & 63) == leader) atomicAdd(&hist[c], (int)__popcll(same));
    todo &= ~same;
  }
}

// ---------------------------------------------------------------- k_sched
constexpr int SCHED_NT = 1024;
constexpr int SCHED_LDS_MAX = 65536;  // bytes of bucket cursors kept in LDS

__global__ __launch_bounds__(SCHED_NT) void k_sched(EaDims d, SeqMeta m,
                                                    const int32_t* __restrict__ unit_cost,
                                                    const int32_t* __restrict__ row_cost,
                                                    const int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ cursor,
                                                    int32_t* __restrict__ sorted_units,
                                                    int64_t* __restrict__ row_off) {
  __shared__ int64_t sm[SCHED_NT / 64 + 1];
  extern __shared__ int32_t lcur[];  // bucket cursors (maxqb + 1), when they fit in LDS
  const bool in_lds = (d.maxqb + 1) * 4 <= SCHED_LDS_MAX;
  int32_t* cur = in_lds ? lcur : cursor;
  const int tid = threadIdx.x;
  const int32_t nb = d.maxqb + 1;  // costs 0..maxqb
  const int32_t nu = m.scal[SCAL_N_UNITS];
  const int64_t nr = (int64_t)nu * d.ngr;
  const int64_t chunk = (nr + SCHED_NT - 1) / SCHED_NT;
  const int64_t r0 = min(nr, tid * chunk), r1 = min(nr, r0 + chunk);
  // Every cost load goes out first, so that their latency overlaps the
  // bucket scan: UPT unit costs and RPT row costs per thread in registers
  // (the rest, on larger batches, loaded where they are used).
  constexpr int UPT = 8, RPT = 16;
  int32_t uc[UPT], rc[RPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int32_t u = tid + i * SCHED_NT;
    uc[i] = u < nu ? unit_cost[u] : 0;
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) rc[i] = r0 + i < r1 ? row_cost[r0 + i] : 0;
  // Bucket starts in descending cost order: cursor[c] = sum_{c' > c} hist[c'].
  {
    const int bchunk = (nb + SCHED_NT - 1) / SCHED_NT;
    const int i0 = min(nb, tid * bchunk), i1 = min(nb, i0 + bchunk);
    int64_t s = 0;
    for (int i = i0; i < i1; ++i) s += hist[d.maxqb - i];
    int64_t tot;
    int64_t e = block_exclusive_sum<SCHED_NT>(s, sm, &tot);
    for (int i = i0; i < i1; ++i) {
      cur[d.maxqb - i] = (int32_t)e;
      e += hist[d.maxqb - i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int32_t u = tid + i * SCHED_NT;
    if (u < nu) sorted_units[atomicAdd(&cur[uc[i]], 1)] = u;
  }
  for (int32_t u = tid + UPT * SCHED_NT; u < nu; u += SCHED_NT) {
    const int32_t pos = atomicAdd(&cur[unit_cost[u]], 1);
    sorted_units[pos] = u;
  }
  // Row offsets into the flat tile list (natural row order).
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) s += rc[i];
  for (int64_t r = r0 + RPT; r < r1; ++r) s += row_cost[r];
  int64_t tot;
  int64_t e = block_exclusive_sum<SCHED_NT>(s, sm, &tot);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    if (r0 + i < r1) row_off[r0 + i] = e;
    e += rc[i];
  }
  for (int64_t r = r0 + RPT; r < r1; ++r) {
    row_off[r] = e;
    e += row_cost[r];
  }
  if (tid == 0) {
    row_off[nr] = tot;
    *(int64_t*)(m.scal + SCAL_TILES64) = tot;
  }
}

// ---------------------------------------------------------------- k_fill
__global__ __launch_bounds__(256) void k_fill(EaDims d, const uint8_t* __restrict__ modes,
                                              const uint32_t* __restrict__ xa_mask, SeqMeta m,
                                              const int32_t* __restrict__ row_cost,
                                              const int64_t* __restrict__ row_off,
                                              uint32_t* __restrict__ tiles) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)m.scal[SCAL_N_UNITS] * d.ngr) return;
  const int64_t u = row / d.ngr;
  const int kg = (int)(row % d.ngr);
  const int32_t qbg = (int32_t)(u / d.Hkv);
  const int g = (int)(u % d.Hkv);
  const int h0 = g * d.G + kg * d.hpw;
  const RowInfo ri = decode_qb(d, m, qbg, g, modes, xa_mask);
  const int64_t off = row_off[row];
  const int32_t cnt = row_cost[row];
  uint32_t* out = tiles + off;
  const uint32_t all_heads = d.hpw == 2 ? (TILE_HEAD0 | (TILE_HEAD0 << 1)) : TILE_HEAD0;
  if (ri.mode == EA_MODE_XA) {
    const uint32_t* mrow = xa_mask + ((int64_t)qbg * d.Hq + h0) * d.words;
    const int nw = ri.I / 32 + 1;
    int32_t base = 0;
    for (int w0 = 0; w0 < nw; w0 += 64) {
      const int w = w0 + lane;
      uint32_t b0 = 0, b1 = 0;
      if (w < nw) {
        const int hi = ri.I - w * 32;
        const uint32_t keep = hi < 31 ? (2u << hi) - 1u : 0xffffffffu;
        b0 = mrow[w] & keep;
        if (d.hpw == 2) b1 = mrow[d.words + w] & keep;
      }
      uint32_t bits = b0 | b1;
      const int32_t pc = __popc(bits);
      const int32_t inc = wave_inclusive_sum(pc);
      int32_t pos = base + inc - pc;
      while (bits) {
        const int t = __ffs(bits) - 1;
        bits &= bits - 1;
        const int32_t J = w * 32 + t;
        const uint32_t hb = (((b0 >> t) & 1u) ? TILE_HEAD0 : 0u) | (((b1 >> t) & 1u) ? (TILE_HEAD0 << 1) : 0u);
        out[pos++] = (uint32_t)J | hb |
                     (tile_needs_mask(d, ri.mode, ri.I, J, ri.len) ? TILE_MASK_FLAG : 0u);
      }
      base += __shfl(inc, 63, 64);
    }
    return;
  }
  int32_t jlo = 0, ns = 0;
  if (ri.mode == EA_MODE_SSA) ssa_ranges(d, ri.I, &jlo, &ns);
  for (int32_t t = lane; t < cnt; t += 64) {
    int32_t J;
    if (ri.mode == EA_MODE_SSA) J = t < ns ? t : jlo + (t - ns);
    else J = t;
    out[t] = (uint32_t)J | all_heads | (tile_needs_mask(d, ri.mode, ri.I, J, ri.len) ? TILE_MASK_FLAG : 0u);
  }
}

hipError_t launch_worklist(const EaDims& d, const uint16_t* k, const uint16_t* v, const uint8_t* modes,
                           const uint32_t* xa_mask, const SeqMeta& m, void* ws, const WsLayout& L,
                           hipStream_t st) {
  char* w = (char*)ws;
  uint16_t* kp = (uint16_t*)(w + L.kvp);
  uint16_t* vp = kp + (size_t)d.Hkv * d.D * (size_t)d.tpad;
  int32_t* unit_cost = (int32_t*)(w + L.unit_cost);
  int32_t* row_cost = (int32_t*)(w + L.row_cost);
  int64_t* row_off = (int64_t*)(w + L.row_off);
  int32_t* hist = (int32_t*)(w + L.hist);
  int32_t* cursor = (int32_t*)(w + L.cursor);
  int32_t* sorted_units = (int32_t*)(w + L.sorted_units);
  uint32_t* tiles = (uint32_t*)(w + L.tiles);
  const dim3 gp((unsigned)d.nqb_max, (unsigned)d.Hkv);
#define EA_PACK(DD, BB) hipLaunchKernelGGL((k_pack<DD, BB>), gp, dim3(256), 0, st, d, k, v, m, kp, vp)
  if (d.D == 128 && d.B == 128) EA_PACK(128, 128);
  else if (d.D == 128 && d.B == 64) EA_PACK(128, 64);
  else if (d.D == 64 && d.B == 128) EA_PACK(64, 128);
  else EA_PACK(64, 64);
#undef EA_PACK
  const int64_t units = d.nqb_max * d.Hkv;
  hipLaunchKernelGGL(k_cost, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, d, modes,
                     xa_mask, m, unit_cost, row_cost, hist);
  const size_t sched_lds = (size_t)(d.maxqb + 1) * 4 <= (size_t)SCHED_LDS_MAX ? (size_t)(d.maxqb + 1) * 4 : 0;
  hipLaunchKernelGGL(k_sched, dim3(1), dim3(SCHED_NT), sched_lds, st, d, m, unit_cost, row_cost, hist,
                     cursor, sorted_units, row_off);
  const int64_t rows = d.nqb_max * d.Hkv * d.ngr;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, d, modes, xa_mask,
                     m, row_cost, row_off, tiles);
  return hipGetLastError();
}

}  // namespace ea
