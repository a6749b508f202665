// Host-only checks of libea's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side (tests/test_host_sanitized.py).
//
// Every call below stays on the host: workspace sizing, mask geometry,
// workspace offsets, status strings, the sparsity ratios, the decode-cache
// layout, and the argument checks of every device entry point (each case is
// rejected before any HIP call, so no GPU is needed).  The sanitizers report
// out-of-bounds accesses and undefined arithmetic (signed overflow, bad
// shifts) in those paths; the program exits non-zero on a wrong status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../include/ea.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static ea_attn_desc desc(int nseq, int T, int maxL, int hq = 32, int hkv = 8, int d = 128, int B = 128) {
  ea_attn_desc a;
  std::memset(&a, 0, sizeof(a));
  a.num_seqs = nseq;
  a.total_tokens = T;
  a.max_seqlen = maxL;
  a.num_q_heads = hq;
  a.num_kv_heads = hkv;
  a.head_dim = d;
  a.block = B;
  a.softmax_scale = 0.088f;
  a.ssa_sink = 128;
  a.ssa_window = 2048;
  a.xa_stride = 8;
  a.xa_tau_num = 9;
  a.xa_tau_den = 10;
  return a;
}

// A 16-byte aligned address that is never dereferenced (every call that
// receives it is rejected before any device work).
static void* const FAKE = reinterpret_cast<void*>(uintptr_t{0x10000});

int main() {
  // 1. Sizing over a grid of descriptors, up to the largest accepted batch.
  const int lens[] = {0, 1, 127, 128, 129, 65536, 262144, 1 << 30, EA_MAX_TOKENS};
  for (int L : lens)
    for (int nseq : {1, 2, 7}) {
      for (int hkv : {1, 8, 64}) {
        const int T = L;
        ea_attn_desc a = desc(nseq, T, T, hkv * 4, hkv);
        for (int op = 0; op <= 3; ++op) {
          const size_t n = ea_workspace_bytes(&a, op);
          if (op != EA_OP_DECODE) EXPECT(n > 0);
        }
        EXPECT(ea_mask_rows(&a) >= 0);
        EXPECT(ea_mask_words(&a) >= 0);
      }
    }
  for (int nseq : {1, 2}) {
    // One token past the limit: no size for any operation.
    ea_attn_desc over = desc(nseq, EA_MAX_TOKENS + 1, EA_MAX_TOKENS + 1);
    for (int op = 0; op <= 3; ++op) EXPECT(ea_workspace_bytes(&over, op) == 0);
  }
  ea_attn_desc bad = desc(1, 100, 100);
  bad.head_dim = 96;
  EXPECT(ea_workspace_bytes(&bad, EA_OP_PREFILL) == 0);
  EXPECT(ea_workspace_bytes(nullptr, EA_OP_PREFILL) == 0);
  EXPECT(ea_workspace_bytes(&bad, 99) == 0);

  // 2. Workspace offsets and status strings.
  const char* names[] = {"seq_start", "seq_len", "qb_prefix", "tri_prefix", "qb2seq", "scal",
                         "xa_pair_bh", "xa_pair_items", "xa_lse", "kvp", "unit_cost", "row_cost",
                         "row_off", "hist", "cursor", "sorted_units", "tiles", "nope", ""};
  ea_attn_desc a = desc(3, 9000, 4000);
  for (const char* n : names)
    for (int op = 0; op <= 3; ++op) (void)ea_workspace_offset(&a, op, n);
  EXPECT(ea_workspace_offset(&a, EA_OP_PREFILL, nullptr) == -1);
  for (int s = -1; s <= 5; ++s) EXPECT(ea_status_string((ea_status)s) != nullptr);

  // 3. Sparsity ratios on random valid batches, then invalid host data.
  std::mt19937 rng(7);
  for (int trial = 0; trial < 200; ++trial) {
    const int nseq = 1 + (int)(rng() % 12), hkv = 1 + (int)(rng() % 8), G = 1 + (int)(rng() % 4);
    std::vector<int32_t> cu(nseq + 1, 0);
    int maxL = 0;
    for (int b = 0; b < nseq; ++b) {
      const int L = (int)(rng() % 3000);
      cu[b + 1] = cu[b] + L;
      maxL = L > maxL ? L : maxL;
    }
    ea_attn_desc r = desc(nseq, cu[nseq], maxL, hkv * G, hkv);
    r.ssa_sink = (int)(rng() % 300);
    r.ssa_window = 1 + (int)(rng() % 4000);
    std::vector<uint8_t> modes(nseq * hkv);
    for (auto& m : modes) m = (uint8_t)(rng() % 3);
    std::vector<int64_t> pairs(nseq * hkv * G);
    for (int b = 0; b < nseq; ++b)
      for (int h = 0; h < hkv * G; ++h) {
        const int64_t L = cu[b + 1] - cu[b];
        pairs[b * hkv * G + h] = L * (L + 1) / 2 / (1 + (int64_t)(rng() % 5));
      }
    std::vector<double> msr(nseq + 1), esr(nseq + 1), rho(nseq * hkv), pw(1);
    EXPECT(ea_sparsity_ratios(&r, cu.data(), modes.data(), 1, pairs.data(), msr.data(), esr.data(),
                              rho.data(), pw.data()) == EA_OK);
    for (int b = 0; b <= nseq; ++b) EXPECT(msr[b] >= 0.0 && msr[b] <= 1.0 && esr[b] >= 0.0 && esr[b] <= 1.0);
    modes[0] = 3;
    EXPECT(ea_sparsity_ratios(&r, cu.data(), modes.data(), 1, pairs.data(), msr.data(), esr.data(),
                              rho.data(), pw.data()) == EA_ERR_INVALID_ARG);
  }

  // 4. Decode-cache layout.
  {
    ea_attn_desc c = desc(3, 3000, 1000, 4, 2);
    c.ssa_sink = 5;
    c.ssa_window = 20;
    uint8_t modes[6] = {0, 1, 1, 2, 1, 1};
    int32_t cap[3] = {1000, 7, 0};
    int64_t seg[7];
    EXPECT(ea_decode_cache_layout(&c, modes, cap, seg) == EA_OK);
    EXPECT(seg[6] == 1039);
    cap[1] = -1;
    EXPECT(ea_decode_cache_layout(&c, modes, cap, seg) == EA_ERR_INVALID_ARG);
  }

  // 5. Every device entry point rejects bad arguments before any device work.
  {
    ea_attn_desc p = desc(1, 4096, 4096);
    const size_t ws = ea_workspace_bytes(&p, EA_OP_PREFILL);
    EXPECT(ea_hybrid_attn_prefill(&p, nullptr, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE,
                                  nullptr, FAKE, (float*)FAKE, FAKE, ws, nullptr) == EA_ERR_INVALID_ARG);
    EXPECT(ea_hybrid_attn_prefill(&p, FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE, nullptr,
                                  FAKE, (float*)FAKE, FAKE, ws - 1, nullptr) == EA_ERR_WORKSPACE);
    EXPECT(ea_hybrid_attn_plan(&p, FAKE, FAKE, nullptr, (const uint8_t*)FAKE, nullptr, FAKE, ws, nullptr) ==
           EA_ERR_INVALID_ARG);
    EXPECT(ea_hybrid_attn_run(&p, FAKE, nullptr, FAKE, (float*)FAKE, FAKE, ws, nullptr) == EA_ERR_INVALID_ARG);
    const size_t wx = ea_workspace_bytes(&p, EA_OP_XA_SELECT);
    EXPECT(ea_xa_block_select(&p, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE, (uint32_t*)FAKE,
                              (int32_t*)FAKE, nullptr, nullptr, FAKE, wx, nullptr) == EA_ERR_INVALID_ARG);
    const size_t wd = ea_workspace_bytes(&p, EA_OP_DECODE);
    EXPECT(ea_hybrid_attn_decode(&p, FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE, FAKE,
                                 (float*)FAKE, FAKE, wd - 1, nullptr) == EA_ERR_WORKSPACE);
    ea_attn_desc big = desc(256, 256 * 65536, 65536);
    EXPECT(ea_hybrid_attn_decode_noalloc(&big, FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE,
                                         FAKE, (float*)FAKE, nullptr) == EA_ERR_WORKSPACE);
    EXPECT(ea_hybrid_attn_decode_cached(&p, FAKE, FAKE, FAKE, nullptr, 10, (const int32_t*)FAKE,
                                        (const uint8_t*)FAKE, FAKE, (float*)FAKE, FAKE, wd, nullptr) ==
           EA_ERR_INVALID_ARG);
    EXPECT(ea_decode_cache_fill(&p, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE,
                                (const int64_t*)FAKE, 0, FAKE, FAKE, nullptr) == EA_ERR_INVALID_ARG);
    EXPECT(ea_decode_cache_append(&p, FAKE, FAKE, (const int32_t*)FAKE, (const uint8_t*)FAKE,
                                  (const int64_t*)FAKE, 10, nullptr, FAKE, nullptr) == EA_ERR_INVALID_ARG);
    uint8_t lm[8] = {0, 1, 2, 0, 1, 1, 0, 1};
    const size_t wsr = ea_workspace_bytes(&p, EA_OP_PREFILL_SERIAL);
    EXPECT(ea_hybrid_attn_prefill_serial(&p, FAKE, FAKE, FAKE, (const int32_t*)FAKE, lm, FAKE, (float*)FAKE,
                                         FAKE, wsr, nullptr) == EA_ERR_UNSUPPORTED);
    ea_router_desc rd;
    std::memset(&rd, 0, sizeof(rd));
    rd.hidden = 3;
    EXPECT(ea_route_heads(&p, &rd, FAKE, (const int32_t*)FAKE, 0, 1, (uint8_t*)FAKE, nullptr, nullptr) ==
           EA_ERR_INVALID_ARG);
  }

  if (failures) {
    std::fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
