// Internal declarations shared by the translation units of libea.so.
//
// Host side: derived sizes (EaDims), the workspace layout, and the launchers
// each .hip file exports.  Device side: small vector types and helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ea.h"

namespace ea {

// Sizes derived from a validated descriptor.  Every bound below depends on
// the descriptor only, so the host can size buffers without reading device
// data (cu_seqlens lives on the device).
struct EaDims {
  int32_t nseq, T, maxL, Hq, Hkv, G, D, B, S, r;  // r = B / S reduced rows per block
  int32_t hpw;      // q-heads per attention workgroup (2 when G is even, else 1)
  int32_t ngr;      // head groups per KV head: G / hpw
  int32_t xa_hpi;   // q-heads per XA scoring item (4, 2 or 1; divides G)
  int32_t xa_group; // 1: one XA mask per KV head (xa_hpi == G)
  int32_t xa_norm;  // 1: P from the raw block sums (softmax per block row)
  float scale;
  int32_t sink, window, tau_num, tau_den;
  int64_t nqb_max;  // bound on sum_b ceil(L_b / B):  T / B + nseq
  int32_t maxqb;    // ceil(maxL / B): bound on q-blocks (and kv-blocks) per sequence
  int32_t words;    // ceil(maxqb / 32): uint32 words per mask row
  int64_t tpad;     // nqb_max * B: padded token count of the packed K / V^T tiles
  int64_t tri_max;  // bound on sum_b nQB_b (nQB_b + 1) / 2
};

// Per-sequence metadata, built on the device from cu_seqlens (sanitised).
struct SeqMeta {
  int32_t* start;       // [nseq] first token
  int32_t* len;         // [nseq] clamped length
  int32_t* qb_prefix;   // [nseq+1] exclusive prefix of ceil(len / B)
  int64_t* tri_prefix;  // [nseq+1] exclusive prefix of nQB (nQB + 1) / 2
  int32_t* qb2seq;      // [nqb_max] global q-block -> sequence
  int32_t* scal;        // [16] scalars, see SCAL_* below
};

enum {
  SCAL_TOTAL_QB = 0,  // sum_b ceil(L_b / B)
  SCAL_XA_PAIRS = 1,  // number of XA (sequence, q-head) pairs that score
  SCAL_N_UNITS = 3,   // total_qb * Hkv
  SCAL_CTR64 = 4,     // int64 work counter of the persistent scoring kernel (words 4..5)
  SCAL_HEAD_TILES64 = 6,  // int64: (tile, q-head) pairs the attention computes (words 6..7)
  SCAL_TILES64 = 8,       // int64: entries of the flat tile list (words 8..9)
  SCAL_COUNT = 16
};

// ---- helpers usable on host and device ----
__host__ __device__ inline int64_t tri64(int64_t n) { return n * (n + 1) / 2; }
// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (no overflow near 2^31).
__host__ __device__ inline int32_t cdiv(int32_t a, int32_t b) { return a / b + (a % b != 0 ? 1 : 0); }

// Byte offsets of every workspace buffer (256-byte aligned).
struct WsLayout {
  size_t seq_start, seq_len, qb_prefix, tri_prefix, qb2seq, scal;
  // XA select
  size_t xa_pair_bh, xa_pair_items, xa_lse;
  // prefill
  size_t kvp, unit_cost, row_cost, row_off, hist, cursor, sorted_units, tiles;
  // decode
  size_t dec_plan, dec_groups, dec_part, dec_ml;
  // serial dispatch: the inner prefill's workspace, then the split copies
  size_t ser_inner, ser_inner_bytes, ser_q, ser_k, ser_v, ser_o, ser_lse, ser_modes;
  size_t total;
};

size_t ws_layout(const EaDims& d, int op, WsLayout* out);
SeqMeta seq_meta_ptrs(const WsLayout& L, void* ws);

// ---- launchers (each returns hipGetLastError() of its launches) ----
hipError_t launch_seq_meta(const EaDims& d, const int32_t* cu, const uint8_t* modes,
                           const SeqMeta& m, void* ws, const WsLayout& L, bool for_select,
                           int64_t* xa_pairs_out, hipStream_t st);
hipError_t launch_xa_score(const EaDims& d, const uint16_t* q, const uint16_t* k,
                           const SeqMeta& m, void* ws, const WsLayout& L, hipStream_t st);
hipError_t launch_xa_select(const EaDims& d, const uint8_t* modes, const SeqMeta& m, void* ws,
                            const WsLayout& L, uint32_t* mask, int32_t* row_count,
                            int64_t* xa_pairs, float* block_mass, hipStream_t st);
hipError_t launch_worklist(const EaDims& d, const uint16_t* k, const uint16_t* v, const uint8_t* modes,
                           const uint32_t* xa_mask, const SeqMeta& m, void* ws,
                           const WsLayout& L, hipStream_t st);
hipError_t launch_attention(const EaDims& d, const uint16_t* q, const uint8_t* modes, const SeqMeta& m, void* ws,
                            const WsLayout& L, uint16_t* o, float* lse, hipStream_t st);
// Decode: kept-key positions per split (one wave each), a power of two in
// [DEC_SPLIT_FLOOR, 4096].  The rule: the smallest split s with
// s * DEC_WAVES >= the step's work, where work = sum over (sequence, KV head)
// of its kept keys times the q-head groups per KV head (G / gw), so the step
// spreads over about DEC_WAVES waves.  Longer splits amortise a wave's
// pipeline start; more splits fill the chip when the batch is small.
// The kept keys depend on the modes, which live in device memory: the host
// bounds the work by the all-FA case (T keys per KV head), which gives the
// largest split.  When that bound leaves a choice, k_decode_plan applies the
// rule to the true work on the device (no lower than an eighth of the bound)
// and lists the workgroups that have work, so no idle one sits between them.
// A workgroup of DEC_WPG waves takes DEC_WPG consecutive splits of one
// (sequence, KV head, head group) and merges them in LDS into one partial,
// so a (sequence, q-head) has cdiv(kept, DEC_WPG * split) partials to combine.
// The grid, the list and the partials are sized for the smallest split.
// With at most DEC_INLINE_UNITS (sequence, KV head, head group) units the
// plan needs no kernel of its own: every wave applies the rule over one
// lane per unit and finds its workgroup's unit by a scan and a ballot.
constexpr int DEC_INLINE_UNITS = 64;
constexpr int32_t DEC_WAVES = 2048;
constexpr int32_t DEC_SPLIT_FLOOR = 64;
constexpr int DEC_WPG = 4;
inline int32_t decode_gw(const EaDims& d) {
  return d.G % 8 == 0 ? 8 : d.G % 4 == 0 ? 4 : d.G % 2 == 0 ? 2 : 1;
}
__host__ __device__ inline int32_t decode_split_rule(int64_t work, int32_t s) {
  while (s < 4096 && (int64_t)s * DEC_WAVES < work) s *= 2;
  return s;
}
inline int32_t decode_split_max(const EaDims& d) {
  return decode_split_rule((int64_t)d.T * d.Hkv * (d.G / decode_gw(d)), DEC_SPLIT_FLOOR);
}
inline int32_t decode_split_min(const EaDims& d) {
  const int32_t s = decode_split_max(d) / 8;
  return s < DEC_SPLIT_FLOOR ? DEC_SPLIT_FLOOR : s;
}
// Partials per (sequence, q-head): one per workgroup of DEC_WPG splits.
inline int32_t decode_parts(const EaDims& d) {
  return (int32_t)(((int64_t)d.maxL + (int64_t)DEC_WPG * decode_split_min(d) - 1) /
                   ((int64_t)DEC_WPG * decode_split_min(d)));
}
// Workgroups of the decode grid: one per (partial, head group, KV head,
// sequence), saturated at 2^62 (the decode call rejects more than 2^31 - 1).
inline int64_t decode_groups(const EaDims& d) {
  const double w = (double)d.nseq * d.Hkv * (d.G / decode_gw(d)) * decode_parts(d);
  return w >= 4.6e18 ? ((int64_t)1 << 62) : (int64_t)d.nseq * d.Hkv * (d.G / decode_gw(d)) * decode_parts(d);
}
// seg == nullptr: k / v are the packed [T, Hkv, D] cache; else the
// segmented head-major cache of cache_rows rows (see ea_decode_cache_layout).
hipError_t launch_decode(const EaDims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* cu, const uint8_t* modes, void* ws, const WsLayout& L,
                         uint16_t* o, float* lse, hipStream_t st, const int64_t* seg = nullptr,
                         int64_t cache_rows = 0);
hipError_t launch_cache_fill(const EaDims& d, const uint16_t* k, const uint16_t* v, const int32_t* cu,
                             const uint8_t* modes, const int64_t* seg, int64_t cache_rows,
                             uint16_t* kc, uint16_t* vc, hipStream_t st);
hipError_t launch_cache_append(const EaDims& d, const uint16_t* kn, const uint16_t* vn, const int32_t* cu,
                               const uint8_t* modes, const int64_t* seg, int64_t cache_rows,
                               uint16_t* kc, uint16_t* vc, hipStream_t st);
// Serial dispatch: head lists (j -> head index) for the split copies.
constexpr int EA_SERIAL_MAX_HEADS = 256;
struct HeadMap {
  int32_t n;
  int32_t idx[EA_SERIAL_MAX_HEADS];
};
hipError_t launch_gather_heads(int D, const uint16_t* src, int32_t hs, uint16_t* dst,
                               const HeadMap& map, int64_t T, hipStream_t st);
hipError_t launch_scatter_heads(int D, const uint16_t* src, const float* lse_src, uint16_t* dst,
                                int32_t hd, float* lse_dst, const HeadMap& map, int64_t T,
                                hipStream_t st);
hipError_t launch_fill_u8(uint8_t* p, int64_t n, uint8_t v, hipStream_t st);
hipError_t launch_route(const EaDims& d, const ea_router_desc& w, const uint16_t* k,
                        const int32_t* cu, uint8_t retrieval_mode, uint8_t sparse_mode,
                        uint8_t* modes, float* logits, hipStream_t st);


// Tile-list entry: kv-block index in bits 0..28, bit 31 = needs a token mask,
// bits 29 and 30 = the first / second q-head of the row's head group attends
// this tile (XA heads of one group may select different blocks).
constexpr uint32_t TILE_MASK_FLAG = 0x80000000u;
constexpr uint32_t TILE_HEAD0 = 0x20000000u;
constexpr uint32_t TILE_J_MASK = 0x1FFFFFFFu;

// Sanitised mode byte: anything but SSA / XA runs as FA.
__host__ __device__ inline int sane_mode(uint8_t m) {
  return (m == EA_MODE_SSA || m == EA_MODE_XA) ? (int)m : (int)EA_MODE_FA;
}

}  // namespace ea
