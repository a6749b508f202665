// C ABI of libea.so: argument validation, workspace layout, launch order,
// and the host-side sparsity ratios.  See include/ea.h for the contract.
#include <cmath>
#include <cstring>
#include <mutex>

#include "ea_internal.h"

namespace ea {

static ea_status make_dims(const ea_attn_desc* desc, EaDims* d) {
  if (!desc) return EA_ERR_INVALID_ARG;
  const ea_attn_desc& a = *desc;
  if (a.num_seqs < 0 || a.total_tokens < 0 || a.max_seqlen < 0) return EA_ERR_INVALID_ARG;
  if (a.num_q_heads < 1 || a.num_kv_heads < 1 || a.num_q_heads % a.num_kv_heads)
    return EA_ERR_INVALID_ARG;
  if (a.num_seqs == 0 && a.total_tokens != 0) return EA_ERR_INVALID_ARG;
  if (a.max_seqlen > a.total_tokens) return EA_ERR_INVALID_ARG;
  if (a.total_tokens > EA_MAX_TOKENS) return EA_ERR_UNSUPPORTED;  // 32-bit token indices in the kernels
  // A valid cu_seqlens needs max_seqlen * num_seqs >= total_tokens.
  if ((int64_t)a.max_seqlen * a.num_seqs < (int64_t)a.total_tokens) return EA_ERR_INVALID_ARG;
  if (!(a.softmax_scale > 0.0f) || !std::isfinite(a.softmax_scale)) return EA_ERR_INVALID_ARG;
  if (a.ssa_sink < 0 || a.ssa_window < 1) return EA_ERR_INVALID_ARG;
  if (a.xa_stride < 1 || a.xa_tau_num < 1 || a.xa_tau_den < 1 || a.xa_tau_num > a.xa_tau_den ||
      a.xa_tau_den > (1 << 20))
    return EA_ERR_INVALID_ARG;
  if (a.xa_group != 0 && a.xa_group != 1) return EA_ERR_INVALID_ARG;
  if (a.xa_norm != 0 && a.xa_norm != 1) return EA_ERR_INVALID_ARG;
  if (a.head_dim != 64 && a.head_dim != 128) return EA_ERR_UNSUPPORTED;
  if (a.block != 64 && a.block != 128) return EA_ERR_UNSUPPORTED;
  if (a.block % a.xa_stride) return EA_ERR_INVALID_ARG;
  const int r = a.block / a.xa_stride;
  if (r != 4 && r != 8 && r != 16 && r != 32) return EA_ERR_UNSUPPORTED;
  d->nseq = a.num_seqs;
  d->T = a.total_tokens;
  d->maxL = a.max_seqlen;
  d->Hq = a.num_q_heads;
  d->Hkv = a.num_kv_heads;
  d->G = a.num_q_heads / a.num_kv_heads;
  d->hpw = (d->G % 2 == 0) ? 2 : 1;
  d->ngr = d->G / d->hpw;
  d->xa_hpi = (d->G % 4 == 0) ? 4 : (d->G % 2 == 0) ? 2 : 1;
  d->xa_group = a.xa_group;
  d->xa_norm = a.xa_norm;
  if (a.xa_group && d->xa_hpi != d->G) return EA_ERR_UNSUPPORTED;
  d->D = a.head_dim;
  d->B = a.block;
  d->S = a.xa_stride;
  d->r = r;
  d->scale = a.softmax_scale;
  d->sink = a.ssa_sink;
  d->window = a.ssa_window;
  d->tau_num = a.xa_tau_num;
  d->tau_den = a.xa_tau_den;
  d->nqb_max = (int64_t)a.total_tokens / a.block + a.num_seqs;
  d->maxqb = cdiv(a.max_seqlen, a.block);
  d->words = cdiv(d->maxqb, 32);
  d->tpad = d->nqb_max * a.block;
  d->tri_max = ((int64_t)(d->maxqb + 1) * d->nqb_max + 1) / 2;
  return EA_OK;
}

static bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ws_layout(const EaDims& d, int op, WsLayout* L) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + (bytes ? bytes : 1));
    return o;
  };
  std::memset(L, 0, sizeof(*L));
  L->seq_start = take(4 * (size_t)d.nseq);
  L->seq_len = take(4 * (size_t)d.nseq);
  L->qb_prefix = take(4 * (size_t)(d.nseq + 1));
  L->tri_prefix = take(8 * (size_t)(d.nseq + 1));
  L->qb2seq = take(4 * (size_t)d.nqb_max);
  L->scal = take(4 * (size_t)SCAL_COUNT);
  if (op == EA_OP_DECODE) {
    if (decode_groups(d) > 0x7fffffff) return 0;  // rejected by the decode call
    const size_t parts = (size_t)d.nseq * d.Hq * (size_t)decode_parts(d);
    L->dec_plan = take(8);
    L->dec_groups = take(8 * (size_t)decode_groups(d));
    L->dec_part = take(4 * parts * d.D);
    L->dec_ml = take(8 * parts);
    L->total = off;
    return off;
  }
  if (op == EA_OP_PREFILL_SERIAL) {
    // The inner single-mode prefills run one after the other on one stream
    // and share a workspace sized for the whole layer (either group needs
    // less); the split copies of q, k, v, o and lse hold both groups.
    WsLayout inner;
    const size_t nb = ws_layout(d, EA_OP_PREFILL, &inner);
    std::memset(L, 0, sizeof(*L));
    off = 0;
    L->ser_inner = take(nb);
    L->ser_inner_bytes = nb;
    const size_t tok = (size_t)d.T;
    L->ser_q = take(2 * tok * d.Hq * d.D);
    L->ser_k = take(2 * tok * d.Hkv * d.D);
    L->ser_v = take(2 * tok * d.Hkv * d.D);
    L->ser_o = take(2 * tok * d.Hq * d.D);
    L->ser_lse = take(4 * tok * d.Hq);
    L->ser_modes = take((size_t)d.nseq * d.Hkv);
    L->total = off;
    return off;
  }
  if (op == EA_OP_XA_SELECT) {
    const size_t pairs = (size_t)d.nseq * d.Hq;
    L->xa_pair_bh = take(4 * pairs);
    L->xa_pair_items = take(8 * (pairs + 1));
    L->xa_lse = take(4 * (size_t)d.r * d.Hq * (size_t)d.tri_max);
  } else {
    const size_t units = (size_t)d.nqb_max * d.Hkv;
    const size_t rows = (size_t)d.nqb_max * d.Hq;
    L->kvp = take(2 * 2 * (size_t)d.Hkv * d.D * (size_t)d.tpad);  // packed K, then V^T
    L->unit_cost = take(4 * units);
    L->row_cost = take(4 * rows);
    L->row_off = take(8 * (rows + 1));
    L->hist = take(4 * (size_t)(d.maxqb + 2));
    L->cursor = take(4 * (size_t)(d.maxqb + 2));
    L->sorted_units = take(4 * units);
    L->tiles = take(4 * (size_t)d.Hq * (size_t)d.tri_max);
  }
  L->total = off;
  return off;
}

SeqMeta seq_meta_ptrs(const WsLayout& L, void* ws) {
  char* b = (char*)ws;
  SeqMeta m;
  m.start = (int32_t*)(b + L.seq_start);
  m.len = (int32_t*)(b + L.seq_len);
  m.qb_prefix = (int32_t*)(b + L.qb_prefix);
  m.tri_prefix = (int64_t*)(b + L.tri_prefix);
  m.qb2seq = (int32_t*)(b + L.qb2seq);
  m.scal = (int32_t*)(b + L.scal);
  return m;
}

}  // namespace ea

using namespace ea;

extern "C" {

size_t ea_workspace_bytes(const ea_attn_desc* desc, int op) {
  EaDims d;
  if (make_dims(desc, &d) != EA_OK) return 0;
  if (op != EA_OP_XA_SELECT && op != EA_OP_PREFILL && op != EA_OP_DECODE &&
      op != EA_OP_PREFILL_SERIAL)
    return 0;
  WsLayout L;
  return ws_layout(d, op, &L);
}

int64_t ea_mask_rows(const ea_attn_desc* desc) {
  EaDims d;
  if (make_dims(desc, &d) != EA_OK) return 0;
  return d.nqb_max * d.Hq;
}

int32_t ea_mask_words(const ea_attn_desc* desc) {
  EaDims d;
  if (make_dims(desc, &d) != EA_OK) return 0;
  return d.words;
}

int64_t ea_workspace_offset(const ea_attn_desc* desc, int op, const char* name) {
  EaDims d;
  if (!name || make_dims(desc, &d) != EA_OK) return -1;
  if (op != EA_OP_XA_SELECT && op != EA_OP_PREFILL) return -1;
  WsLayout L;
  ws_layout(d, op, &L);
  // which: 0 = both operations, 1 = XA select only, 2 = prefill only
  struct { const char* n; int which; size_t o; } tab[] = {
      {"seq_start", 0, L.seq_start},   {"seq_len", 0, L.seq_len},
      {"qb_prefix", 0, L.qb_prefix},   {"tri_prefix", 0, L.tri_prefix},
      {"qb2seq", 0, L.qb2seq},         {"scal", 0, L.scal},
      {"xa_pair_bh", 1, L.xa_pair_bh}, {"xa_pair_items", 1, L.xa_pair_items},
      {"xa_lse", 1, L.xa_lse},         {"kvp", 2, L.kvp},
      {"unit_cost", 2, L.unit_cost},   {"row_cost", 2, L.row_cost},
      {"row_off", 2, L.row_off},       {"hist", 2, L.hist},
      {"cursor", 2, L.cursor},         {"sorted_units", 2, L.sorted_units},
      {"tiles", 2, L.tiles}};
  const int want = op == EA_OP_XA_SELECT ? 1 : 2;
  for (auto& e : tab)
    if (std::strcmp(e.n, name) == 0) return (e.which == 0 || e.which == want) ? (int64_t)e.o : -1;
  return -1;
}

const char* ea_status_string(ea_status s) {
  // A C caller may pass any int: read the argument's bytes instead of loading
  // it as the enum (out-of-range enum values are undefined behaviour in C++).
  int v;
  static_assert(sizeof(v) == sizeof(s), "ea_status is int-sized");
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case EA_OK: return "EA_OK";
    case EA_ERR_INVALID_ARG: return "EA_ERR_INVALID_ARG: invalid argument";
    case EA_ERR_UNSUPPORTED: return "EA_ERR_UNSUPPORTED: configuration not built";
    case EA_ERR_WORKSPACE: return "EA_ERR_WORKSPACE: workspace missing or too small";
    case EA_ERR_HIP: return "EA_ERR_HIP: a HIP launch failed";
  }
  return "unknown ea_status";
}

ea_status ea_xa_block_select(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                             const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                             uint32_t* mask_out_dev, int32_t* row_count_out_dev,
                             int64_t* xa_pairs_out_dev, float* block_mass_out_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!cu_seqlens_dev || !modes_dev || !xa_pairs_out_dev) return EA_ERR_INVALID_ARG;
  if (d.T > 0 && (!q_dev || !k_dev || !mask_out_dev || !row_count_out_dev))
    return EA_ERR_INVALID_ARG;
  if (misaligned(q_dev) || misaligned(k_dev)) return EA_ERR_INVALID_ARG;
  // The selector keeps one block row (mass + weight) in LDS.
  if ((int64_t)d.maxqb * 8 > 96 * 1024) return EA_ERR_UNSUPPORTED;
  WsLayout L;
  const size_t need = ws_layout(d, EA_OP_XA_SELECT, &L);
  if (!workspace_dev || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (d.nseq == 0) return EA_OK;
  hipStream_t s = (hipStream_t)stream;
  SeqMeta m = seq_meta_ptrs(L, workspace_dev);
  if (launch_seq_meta(d, cu_seqlens_dev, modes_dev, m, workspace_dev, L, true, xa_pairs_out_dev, s) !=
      hipSuccess)
    return EA_ERR_HIP;
  if (d.T == 0) return EA_OK;
  if (launch_xa_score(d, (const uint16_t*)q_dev, (const uint16_t*)k_dev, m, workspace_dev, L, s) !=
      hipSuccess)
    return EA_ERR_HIP;
  if (launch_xa_select(d, modes_dev, m, workspace_dev, L, mask_out_dev, row_count_out_dev,
                       xa_pairs_out_dev, block_mass_out_dev, s) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_hybrid_attn_plan(const ea_attn_desc* desc, const void* k_dev, const void* v_dev,
                              const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                              const uint32_t* xa_mask_dev, void* workspace_dev,
                              size_t workspace_bytes, void* stream) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!cu_seqlens_dev || !modes_dev) return EA_ERR_INVALID_ARG;
  if (d.T > 0 && (!k_dev || !v_dev)) return EA_ERR_INVALID_ARG;
  if (misaligned(k_dev) || misaligned(v_dev)) return EA_ERR_INVALID_ARG;
  WsLayout L;
  const size_t need = ws_layout(d, EA_OP_PREFILL, &L);
  if (!workspace_dev || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (d.T == 0) return EA_OK;
  hipStream_t s = (hipStream_t)stream;
  SeqMeta m = seq_meta_ptrs(L, workspace_dev);
  if (launch_seq_meta(d, cu_seqlens_dev, modes_dev, m, workspace_dev, L, false, nullptr, s) !=
      hipSuccess)
    return EA_ERR_HIP;
  if (launch_worklist(d, (const uint16_t*)k_dev, (const uint16_t*)v_dev, modes_dev, xa_mask_dev,
                      m, workspace_dev, L, s) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_hybrid_attn_run(const ea_attn_desc* desc, const void* q_dev,
                             const uint8_t* modes_dev, void* o_out_dev, float* lse_out_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!modes_dev) return EA_ERR_INVALID_ARG;
  if (d.T > 0 && (!q_dev || !o_out_dev || !lse_out_dev)) return EA_ERR_INVALID_ARG;
  if (misaligned(q_dev) || misaligned(o_out_dev)) return EA_ERR_INVALID_ARG;
  WsLayout L;
  const size_t need = ws_layout(d, EA_OP_PREFILL, &L);
  if (!workspace_dev || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (d.T == 0) return EA_OK;
  SeqMeta m = seq_meta_ptrs(L, workspace_dev);
  if (launch_attention(d, (const uint16_t*)q_dev, modes_dev, m, workspace_dev, L,
                       (uint16_t*)o_out_dev, lse_out_dev, (hipStream_t)stream) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_hybrid_attn_prefill(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                                 const void* v_dev, const int32_t* cu_seqlens_dev,
                                 const uint8_t* modes_dev, const uint32_t* xa_mask_dev,
                                 void* o_out_dev, float* lse_out_dev, void* workspace_dev,
                                 size_t workspace_bytes, void* stream) {
  // Validate everything before the first launch: run's checks are made here
  // too, so a bad q / o / lse never leaves a half-done plan behind.
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (d.T > 0 && (!q_dev || !o_out_dev || !lse_out_dev)) return EA_ERR_INVALID_ARG;
  if (misaligned(q_dev) || misaligned(o_out_dev)) return EA_ERR_INVALID_ARG;
  st = ea_hybrid_attn_plan(desc, k_dev, v_dev, cu_seqlens_dev, modes_dev, xa_mask_dev,
                           workspace_dev, workspace_bytes, stream);
  if (st != EA_OK) return st;
  return ea_hybrid_attn_run(desc, q_dev, modes_dev, o_out_dev, lse_out_dev, workspace_dev,
                            workspace_bytes, stream);
}

ea_status ea_hybrid_attn_prefill_serial(const ea_attn_desc* desc, const void* q_dev,
                                        const void* k_dev, const void* v_dev,
                                        const int32_t* cu_seqlens_dev,
                                        const uint8_t* layer_modes_host, void* o_out_dev,
                                        float* lse_out_dev, void* workspace_dev,
                                        size_t workspace_bytes, void* stream) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!cu_seqlens_dev || !layer_modes_host) return EA_ERR_INVALID_ARG;
  if (d.T > 0 && (!q_dev || !k_dev || !v_dev || !o_out_dev || !lse_out_dev))
    return EA_ERR_INVALID_ARG;
  if (misaligned(q_dev) || misaligned(k_dev) || misaligned(v_dev) || misaligned(o_out_dev) ||
      ((uintptr_t)lse_out_dev & 3u))
    return EA_ERR_INVALID_ARG;
  for (int g = 0; g < d.Hkv; ++g) {
    if (layer_modes_host[g] > EA_MODE_XA) return EA_ERR_INVALID_ARG;
    if (layer_modes_host[g] == EA_MODE_XA) return EA_ERR_UNSUPPORTED;
  }
  if (d.Hq > EA_SERIAL_MAX_HEADS) return EA_ERR_UNSUPPORTED;
  WsLayout L;
  const size_t need = ws_layout(d, EA_OP_PREFILL_SERIAL, &L);
  if (!workspace_dev || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (d.T == 0) return EA_OK;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)workspace_dev;
  // 1. Split: the KV heads of each mode and their q-heads, copied into
  //    contiguous tensors of their own (full group first).
  HeadMap kmap[2], qmap[2];
  for (int grp = 0; grp < 2; ++grp) {
    kmap[grp].n = qmap[grp].n = 0;
    const uint8_t mode = grp == 0 ? EA_MODE_FA : EA_MODE_SSA;
    for (int g = 0; g < d.Hkv; ++g)
      if (layer_modes_host[g] == mode) {
        kmap[grp].idx[kmap[grp].n++] = g;
        for (int u = 0; u < d.G; ++u) qmap[grp].idx[qmap[grp].n++] = g * d.G + u;
      }
  }
  const int64_t T = d.T;
  uint16_t* qs[2];
  uint16_t* ks[2];
  uint16_t* vs[2];
  uint16_t* os[2];
  float* ls[2];
  uint8_t* ms[2];
  for (int grp = 0; grp < 2; ++grp) {
    const int64_t hq0 = grp == 0 ? 0 : qmap[0].n, hk0 = grp == 0 ? 0 : kmap[0].n;
    qs[grp] = (uint16_t*)(w + L.ser_q) + T * hq0 * d.D;
    ks[grp] = (uint16_t*)(w + L.ser_k) + T * hk0 * d.D;
    vs[grp] = (uint16_t*)(w + L.ser_v) + T * hk0 * d.D;
    os[grp] = (uint16_t*)(w + L.ser_o) + T * hq0 * d.D;
    ls[grp] = (float*)(w + L.ser_lse) + T * hq0;
    ms[grp] = (uint8_t*)(w + L.ser_modes) + (int64_t)d.nseq * hk0;
  }
  for (int grp = 0; grp < 2; ++grp) {
    if (kmap[grp].n == 0) continue;
    if (launch_gather_heads(d.D, (const uint16_t*)q_dev, d.Hq, qs[grp], qmap[grp], T, s) != hipSuccess ||
        launch_gather_heads(d.D, (const uint16_t*)k_dev, d.Hkv, ks[grp], kmap[grp], T, s) != hipSuccess ||
        launch_gather_heads(d.D, (const uint16_t*)v_dev, d.Hkv, vs[grp], kmap[grp], T, s) != hipSuccess ||
        launch_fill_u8(ms[grp], (int64_t)d.nseq * kmap[grp].n, grp == 0 ? EA_MODE_FA : EA_MODE_SSA, s) !=
            hipSuccess)
      return EA_ERR_HIP;
  }
  // 2. One single-mode layer per group: all-FA, then all-SSA.
  for (int grp = 0; grp < 2; ++grp) {
    if (kmap[grp].n == 0) continue;
    ea_attn_desc sub = *desc;
    sub.num_kv_heads = kmap[grp].n;
    sub.num_q_heads = qmap[grp].n;
    st = ea_hybrid_attn_prefill(&sub, qs[grp], ks[grp], vs[grp], cu_seqlens_dev, ms[grp], nullptr,
                                os[grp], ls[grp], w + L.ser_inner, L.ser_inner_bytes, stream);
    if (st != EA_OK) return st;
  }
  // 3. Write both groups back into the layer's o and lse.
  for (int grp = 0; grp < 2; ++grp) {
    if (kmap[grp].n == 0) continue;
    if (launch_scatter_heads(d.D, os[grp], ls[grp], (uint16_t*)o_out_dev, d.Hq, lse_out_dev, qmap[grp],
                             T, s) != hipSuccess)
      return EA_ERR_HIP;
  }
  return EA_OK;
}

}  // extern "C"

namespace ea {

// Host-side checks of a decode step, shared by the two decode entry points.
static ea_status decode_check(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                              const void* v_dev, const int32_t* cu_seqlens_dev,
                              const uint8_t* modes_dev, void* o_out_dev, float* lse_out_dev,
                              EaDims* d, WsLayout* L, size_t* need) {
  ea_status st = make_dims(desc, d);
  if (st != EA_OK) return st;
  if (d->G > 16) return EA_ERR_UNSUPPORTED;
  if (!cu_seqlens_dev || !modes_dev) return EA_ERR_INVALID_ARG;
  if (d->nseq > 0 && (!q_dev || !o_out_dev || !lse_out_dev)) return EA_ERR_INVALID_ARG;
  if (d->T > 0 && (!k_dev || !v_dev)) return EA_ERR_INVALID_ARG;
  if (misaligned(q_dev) || misaligned(k_dev) || misaligned(v_dev) || misaligned(o_out_dev) ||
      ((uintptr_t)lse_out_dev & 3u))
    return EA_ERR_INVALID_ARG;
  if (d->nseq > 65535 || d->Hkv > 65535) return EA_ERR_UNSUPPORTED;
  if (decode_groups(*d) > 0x7fffffff) return EA_ERR_UNSUPPORTED;
  *need = ws_layout(*d, EA_OP_DECODE, L);
  return EA_OK;
}

// Scratch of ea_hybrid_attn_decode_noalloc: the library's own device memory,
// one copy per GPU (each at its own address), held until the process ends.
// Host code never uses the array's name as an address: the device address
// of the current GPU's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[EA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices];

static ea_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return EA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return EA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EA_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return EA_OK;
}

}  // namespace ea

extern "C" {

ea_status ea_hybrid_attn_decode(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                                const void* v_dev, const int32_t* cu_seqlens_dev,
                                const uint8_t* modes_dev, void* o_out_dev, float* lse_out_dev,
                                void* workspace_dev, size_t workspace_bytes, void* stream) {
  EaDims d;
  WsLayout L;
  size_t need = 0;
  ea_status st = decode_check(desc, q_dev, k_dev, v_dev, cu_seqlens_dev, modes_dev, o_out_dev,
                              lse_out_dev, &d, &L, &need);
  if (st != EA_OK) return st;
  if (!workspace_dev || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (d.nseq == 0) return EA_OK;
  if (launch_decode(d, (const uint16_t*)q_dev, (const uint16_t*)k_dev, (const uint16_t*)v_dev,
                    cu_seqlens_dev, modes_dev, workspace_dev, L,
                    (uint16_t*)o_out_dev, lse_out_dev, (hipStream_t)stream) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_decode_cache_layout(const ea_attn_desc* desc, const uint8_t* modes_host,
                                 const int32_t* capacity_host, int64_t* seg_off_host) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!seg_off_host || (d.nseq > 0 && (!modes_host || !capacity_host))) return EA_ERR_INVALID_ARG;
  for (int b = 0; b < d.nseq; ++b) {
    if (capacity_host[b] < 0) return EA_ERR_INVALID_ARG;
    for (int g = 0; g < d.Hkv; ++g)
      if (modes_host[(size_t)b * d.Hkv + g] > EA_MODE_XA) return EA_ERR_INVALID_ARG;
  }
  const int64_t ring = (int64_t)d.sink + d.window;
  int64_t off = 0;
  seg_off_host[0] = 0;
  for (int b = 0; b < d.nseq; ++b)
    for (int g = 0; g < d.Hkv; ++g) {
      const int64_t cap = capacity_host[b];
      const bool ssa = modes_host[(size_t)b * d.Hkv + g] == EA_MODE_SSA;
      off += ssa ? (cap < ring ? cap : ring) : cap;
      seg_off_host[(size_t)b * d.Hkv + g + 1] = off;
    }
  return EA_OK;
}

static ea_status cache_check(const ea_attn_desc* desc, EaDims* d, const void* a_dev, const void* b_dev,
                             const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                             const int64_t* seg_off_dev, int64_t cache_rows, const void* kc,
                             const void* vc) {
  ea_status st = make_dims(desc, d);
  if (st != EA_OK) return st;
  if (!cu_seqlens_dev || !modes_dev || !seg_off_dev || cache_rows < 0) return EA_ERR_INVALID_ARG;
  if (d->T > 0 && (!a_dev || !b_dev || !kc || !vc || cache_rows < 1)) return EA_ERR_INVALID_ARG;
  if (misaligned(a_dev) || misaligned(b_dev) || misaligned(kc) || misaligned(vc)) return EA_ERR_INVALID_ARG;
  if ((int64_t)d->nseq * d->Hkv > 65535) return EA_ERR_UNSUPPORTED;
  return EA_OK;
}

ea_status ea_decode_cache_fill(const ea_attn_desc* desc, const void* k_dev, const void* v_dev,
                               const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                               const int64_t* seg_off_dev, int64_t cache_rows, void* k_cache_dev,
                               void* v_cache_dev, void* stream) {
  EaDims d;
  ea_status st = cache_check(desc, &d, k_dev, v_dev, cu_seqlens_dev, modes_dev, seg_off_dev, cache_rows,
                             k_cache_dev, v_cache_dev);
  if (st != EA_OK) return st;
  if (d.T == 0 || d.nseq == 0) return EA_OK;
  if (launch_cache_fill(d, (const uint16_t*)k_dev, (const uint16_t*)v_dev, cu_seqlens_dev, modes_dev,
                        seg_off_dev, cache_rows, (uint16_t*)k_cache_dev, (uint16_t*)v_cache_dev,
                        (hipStream_t)stream) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_decode_cache_append(const ea_attn_desc* desc, const void* k_new_dev,
                                 const void* v_new_dev, const int32_t* cu_seqlens_dev,
                                 const uint8_t* modes_dev, const int64_t* seg_off_dev,
                                 int64_t cache_rows, void* k_cache_dev, void* v_cache_dev,
                                 void* stream) {
  EaDims d;
  ea_status st = cache_check(desc, &d, k_new_dev, v_new_dev, cu_seqlens_dev, modes_dev, seg_off_dev,
                             cache_rows, k_cache_dev, v_cache_dev);
  if (st != EA_OK) return st;
  if (d.T == 0 || d.nseq == 0) return EA_OK;
  if (launch_cache_append(d, (const uint16_t*)k_new_dev, (const uint16_t*)v_new_dev, cu_seqlens_dev,
                          modes_dev, seg_off_dev, cache_rows, (uint16_t*)k_cache_dev,
                          (uint16_t*)v_cache_dev, (hipStream_t)stream) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_hybrid_attn_decode_cached(const ea_attn_desc* desc, const void* q_dev,
                                       const void* k_cache_dev, const void* v_cache_dev,
                                       const int64_t* seg_off_dev, int64_t cache_rows,
                                       const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                                       void* o_out_dev, float* lse_out_dev, void* workspace_dev,
                                       size_t workspace_bytes, void* stream) {
  EaDims d;
  WsLayout L;
  size_t need = 0;
  ea_status st = decode_check(desc, q_dev, k_cache_dev, v_cache_dev, cu_seqlens_dev, modes_dev,
                              o_out_dev, lse_out_dev, &d, &L, &need);
  if (st != EA_OK) return st;
  if (!seg_off_dev || cache_rows < 0 || (d.T > 0 && cache_rows < 1)) return EA_ERR_INVALID_ARG;
  if (!workspace_dev || workspace_bytes < need) return EA_ERR_WORKSPACE;
  if (d.nseq == 0) return EA_OK;
  if (launch_decode(d, (const uint16_t*)q_dev, (const uint16_t*)k_cache_dev,
                    (const uint16_t*)v_cache_dev, cu_seqlens_dev, modes_dev, workspace_dev, L,
                    (uint16_t*)o_out_dev, lse_out_dev, (hipStream_t)stream, seg_off_dev,
                    cache_rows) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_hybrid_attn_decode_noalloc(const ea_attn_desc* desc, const void* q_dev,
                                        const void* k_dev, const void* v_dev,
                                        const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                                        void* o_out_dev, float* lse_out_dev, void* stream) {
  EaDims d;
  WsLayout L;
  size_t need = 0;
  ea_status st = decode_check(desc, q_dev, k_dev, v_dev, cu_seqlens_dev, modes_dev, o_out_dev,
                              lse_out_dev, &d, &L, &need);
  if (st != EA_OK) return st;
  if (need > (size_t)EA_DECODE_NOALLOC_SCRATCH_BYTES) return EA_ERR_WORKSPACE;
  if (d.nseq == 0) return EA_OK;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != EA_OK) return st;
  // Nothing in the scratch has to start at zero: the split is written by
  // k_decode_plan (with the workgroup list) or, for steps of at most 64
  // units, by the first k_decode workgroup, and the combine reads only the
  // partials that this step's own workgroups wrote.
  if (launch_decode(d, (const uint16_t*)q_dev, (const uint16_t*)k_dev, (const uint16_t*)v_dev,
                    cu_seqlens_dev, modes_dev, ws, L, (uint16_t*)o_out_dev, lse_out_dev,
                    (hipStream_t)stream) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_route_heads(const ea_attn_desc* desc, const ea_router_desc* router,
                         const void* k_dev, const int32_t* cu_seqlens_dev,
                         uint8_t retrieval_mode, uint8_t sparse_mode, uint8_t* modes_out_dev,
                         float* logits_out_dev, void* stream) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!router || !cu_seqlens_dev) return EA_ERR_INVALID_ARG;
  const ea_router_desc& w = *router;
  if (w.hidden < 4 || w.hidden > 1024 || w.hidden % 4 || w.pool_head < 0 || w.pool_tail < 0)
    return EA_ERR_INVALID_ARG;
  if (retrieval_mode > 2 || sparse_mode > 2) return EA_ERR_INVALID_ARG;
  if (d.nseq == 0) return EA_OK;
  if (!modes_out_dev || !w.w1 || !w.b1 || !w.w2 || !w.b2 || !w.w3 || !w.b3 || !w.w4 || !w.b4)
    return EA_ERR_INVALID_ARG;
  const void* wp[8] = {w.w1, w.b1, w.w2, w.b2, w.w3, w.b3, w.w4, w.b4};
  for (const void* p : wp)
    if ((uintptr_t)p & 3u) return EA_ERR_INVALID_ARG;
  if (misaligned(w.w1) || misaligned(w.w2) || misaligned(w.w3)) return EA_ERR_INVALID_ARG;
  if (d.T > 0 && !k_dev) return EA_ERR_INVALID_ARG;
  if (misaligned(k_dev) || ((uintptr_t)logits_out_dev & 3u)) return EA_ERR_INVALID_ARG;
  if ((int64_t)d.nseq * d.Hkv > 0x7fffffff) return EA_ERR_UNSUPPORTED;
  if (launch_route(d, w, (const uint16_t*)k_dev, cu_seqlens_dev, retrieval_mode, sparse_mode,
                   modes_out_dev, logits_out_dev, (hipStream_t)stream) != hipSuccess)
    return EA_ERR_HIP;
  return EA_OK;
}

ea_status ea_sparsity_ratios(const ea_attn_desc* desc, const int32_t* cu, const uint8_t* modes,
                             uint8_t sparse_mode, const int64_t* xa_pairs, double* msr_out,
                             double* esr_out, double* rho_out, double* esr_pw_out) {
  EaDims d;
  ea_status st = make_dims(desc, &d);
  if (st != EA_OK) return st;
  if (!cu || !modes || !msr_out || !esr_out || !rho_out) return EA_ERR_INVALID_ARG;
  if (sparse_mode > 2) return EA_ERR_INVALID_ARG;
  const int nseq = d.nseq, Hkv = d.Hkv, G = d.G;
  if (cu[0] != 0 || cu[nseq] != d.T) return EA_ERR_INVALID_ARG;
  bool any_xa = false;
  for (int b = 0; b < nseq; ++b) {
    const int64_t L = (int64_t)cu[b + 1] - cu[b];
    if (L < 0 || L > d.maxL) return EA_ERR_INVALID_ARG;
    for (int g = 0; g < Hkv; ++g) {
      const uint8_t mo = modes[(size_t)b * Hkv + g];
      if (mo > 2) return EA_ERR_INVALID_ARG;
      if (mo == EA_MODE_XA) any_xa = true;
    }
  }
  if (any_xa && !xa_pairs) return EA_ERR_INVALID_ARG;
  // Validate XA pair counts before writing anything.
  for (int b = 0; b < nseq && any_xa; ++b) {
    const int64_t L = (int64_t)cu[b + 1] - cu[b];
    for (int h = 0; h < d.Hq; ++h)
      if (modes[(size_t)b * Hkv + h / G] == EA_MODE_XA) {
        const int64_t p = xa_pairs[(size_t)b * d.Hq + h];
        if (p < 0 || p > tri64(L)) return EA_ERR_INVALID_ARG;
      }
  }
  double kept_tot = 0.0, causal_tot = 0.0;
  double msr_sum = 0.0, esr_sum = 0.0;
  for (int b = 0; b < nseq; ++b) {
    const int64_t L = (int64_t)cu[b + 1] - cu[b];
    const int64_t causal = tri64(L);
    // SSA kept pairs: per query, |{j < sink, j <= i}| + |window part outside the sink|.
    int64_t ssa = 0;
    bool need_ssa = false;
    for (int g = 0; g < Hkv; ++g) need_ssa |= modes[(size_t)b * Hkv + g] == EA_MODE_SSA;
    if (need_ssa)
      for (int64_t i = 0; i < L; ++i) {
        const int64_t ns = i + 1 < d.sink ? i + 1 : d.sink;
        int64_t lo = i - d.window + 1;
        if (lo < 0) lo = 0;
        const int64_t from = lo > d.sink ? lo : d.sink;
        ssa += ns + (i - from + 1 > 0 ? i - from + 1 : 0);
      }
    double rs = 0.0;
    int nsparse = 0;
    for (int g = 0; g < Hkv; ++g) {
      const uint8_t mo = modes[(size_t)b * Hkv + g];
      int64_t kept;
      if (mo == EA_MODE_FA) kept = (int64_t)G * causal;
      else if (mo == EA_MODE_SSA) kept = (int64_t)G * ssa;
      else {
        kept = 0;
        for (int h = g * G; h < (g + 1) * G; ++h) kept += xa_pairs[(size_t)b * d.Hq + h];
      }
      const double rho = causal == 0 ? 0.0 : 1.0 - (double)kept / ((double)G * (double)causal);
      rho_out[(size_t)b * Hkv + g] = rho;
      rs += rho;
      nsparse += (mo == sparse_mode);
      kept_tot += (double)kept;
      causal_tot += (double)G * (double)causal;
    }
    msr_out[b] = (double)nsparse / Hkv;
    esr_out[b] = rs / Hkv;
    msr_sum += msr_out[b];
    esr_sum += esr_out[b];
  }
  msr_out[nseq] = nseq ? msr_sum / nseq : 0.0;
  esr_out[nseq] = nseq ? esr_sum / nseq : 0.0;
  if (esr_pw_out) *esr_pw_out = causal_tot == 0.0 ? 0.0 : 1.0 - kept_tot / causal_tot;
  return EA_OK;
}

}  // extern "C"
