// Per-sequence metadata: sanitised lengths, q-block prefixes, the q-block ->
// sequence map and (for XA selection) the compact list of scoring pairs.
#include "ea_device.h"

namespace ea {

constexpr int META_NT = 1024;
constexpr int XA_TILE = 128;  // reduced rows / columns per scoring tile

__global__ __launch_bounds__(META_NT) void k_seq_meta(EaDims d, const int32_t* __restrict__ cu,
                                                      const uint8_t* __restrict__ modes, SeqMeta m,
                                                      int32_t* pair_bh, int64_t* pair_items,
                                                      int64_t* xa_pairs_out, int32_t* hist,
                                                      int for_select) {
  __shared__ int64_t sm[META_NT / 64 + 1];
  const int tid = threadIdx.x;
  const int nseq = d.nseq;

  // 1. Sanitised (start, len) per sequence; each thread owns a contiguous chunk.
  //    start_b = max(clamp(cu[b]), max_{b' < b} end_b'), end_b = clamp(cu[b+1])
  //    with len_b <= max_seqlen: the sequences are disjoint and inside [0, T),
  //    whatever cu_seqlens holds, and equal to cu_seqlens when it is valid.
  const int chunk = cdiv(nseq, META_NT);
  const int b0 = min(nseq, tid * chunk), b1 = min(nseq, b0 + chunk);
  int64_t emax = 0;
  for (int b = b0; b < b1; ++b) {
    const int64_t s0 = min<int64_t>(max<int64_t>(cu[b], 0), d.T);
    int64_t e0 = min<int64_t>(max<int64_t>(cu[b + 1], 0), d.T);
    e0 = min<int64_t>(max(e0, s0), s0 + d.maxL);
    emax = max(emax, e0);
  }
  int64_t prev_end = block_exclusive_max<META_NT>(emax, (int64_t)0, sm);
  int64_t sq = 0, st = 0;
  for (int b = b0; b < b1; ++b) {
    const int64_t s0 = min<int64_t>(max<int64_t>(cu[b], 0), d.T);
    int64_t e0 = min<int64_t>(max<int64_t>(cu[b + 1], 0), d.T);
    e0 = min<int64_t>(max(e0, s0), s0 + d.maxL);
    const int64_t start = max(s0, prev_end);
    const int32_t len = (int32_t)max<int64_t>(0, e0 - start);
    prev_end = max(prev_end, e0);
    m.start[b] = (int32_t)start;
    m.len[b] = len;
    const int32_t nqb = cdiv(len, d.B);
    sq += nqb;
    st += tri64(nqb);
  }
  int64_t totq, tott;
  int64_t eq = block_exclusive_sum<META_NT>(sq, sm, &totq);
  int64_t et = block_exclusive_sum<META_NT>(st, sm, &tott);
  for (int b = b0; b < b1; ++b) {
    const int32_t nqb = cdiv(m.len[b], d.B);
    m.qb_prefix[b] = (int32_t)eq;
    m.tri_prefix[b] = et;
    eq += nqb;
    et += tri64(nqb);
  }
  if (tid == 0) {
    m.qb_prefix[nseq] = (int32_t)totq;
    m.tri_prefix[nseq] = tott;
    m.scal[SCAL_TOTAL_QB] = (int32_t)totq;
    m.scal[SCAL_N_UNITS] = (int32_t)(totq * d.Hkv);
    m.scal[SCAL_XA_PAIRS] = 0;
    for (int i = SCAL_CTR64; i < SCAL_COUNT; ++i) m.scal[i] = 0;
  }
  __syncthreads();

  // 2. Global q-block -> sequence (empty sequences own no block).
  for (int64_t q = tid; q < totq; q += META_NT)
    m.qb2seq[q] = upper_index(m.qb_prefix, nseq + 1, (int32_t)q);

  if (!for_select) {
    for (int c = tid; c < d.maxqb + 2; c += META_NT) hist[c] = 0;
    return;
  }

  // 3. XA scoring pairs (sequence, group of xa_hpi q-heads of one KV head) in
  //    (b, group) order, with the prefix of their triangular tile counts; zero
  //    the attended-pair counters of every (sequence, q-head).
  for (int64_t p = tid; p < (int64_t)nseq * d.Hq; p += META_NT) xa_pairs_out[p] = 0;
  const int nhg = d.Hq / d.xa_hpi;
  const int64_t np = (int64_t)nseq * nhg;
  const int64_t c2 = (np + META_NT - 1) / META_NT;
  const int64_t p0 = min(np, tid * c2), p1 = min(np, p0 + c2);
  int64_t cnt = 0, items = 0;
  auto is_xa = [&](int64_t p) {
    const int b = (int)(p / nhg), g = (int)(p % nhg) * d.xa_hpi / d.G;
    const int32_t len = m.len[b];
    return sane_mode(modes[(int64_t)b * d.Hkv + g]) == EA_MODE_XA && len > 0 && len % d.B == 0;
  };
  for (int64_t p = p0; p < p1; ++p) {
    if (is_xa(p)) {
      cnt += 1;
      items += tri64(cdiv(m.len[p / nhg] / d.S, XA_TILE));
    }
  }
  int64_t totc, toti;
  int64_t ec = block_exclusive_sum<META_NT>(cnt, sm, &totc);
  int64_t ei = block_exclusive_sum<META_NT>(items, sm, &toti);
  for (int64_t p = p0; p < p1; ++p) {
    if (is_xa(p)) {
      pair_bh[ec] = (int32_t)p;
      pair_items[ec] = ei;
      ec += 1;
      ei += tri64(cdiv(m.len[p / nhg] / d.S, XA_TILE));
    }
  }
  if (tid == 0) {
    pair_items[totc] = toti;
    m.scal[SCAL_XA_PAIRS] = (int32_t)totc;
  }
}

hipError_t launch_seq_meta(const EaDims& d, const int32_t* cu, const uint8_t* modes,
                           const SeqMeta& m, void* ws, const WsLayout& L, bool for_select,
                           int64_t* xa_pairs_out, hipStream_t st) {
  char* w = (char*)ws;
  int32_t* pair_bh = for_select ? (int32_t*)(w + L.xa_pair_bh) : nullptr;
  int64_t* pair_items = for_select ? (int64_t*)(w + L.xa_pair_items) : nullptr;
  int32_t* hist = for_select ? nullptr : (int32_t*)(w + L.hist);
  hipLaunchKernelGGL(k_seq_meta, dim3(1), dim3(META_NT), 0, st, d, cu, modes, m, pair_bh,
                     pair_items, xa_pairs_out, hist, for_select ? 1 : 0);
  return hipGetLastError();
}

}  // namespace ea
