// Drives the host side of the C ABI (include/duo.h) built with
// AddressSanitizer and UndefinedBehaviorSanitizer against stand-in launchers:
// layouts, descriptor and argument validation, token counts, ragged views and
// their workspace offsets, failure handling, and the host helpers. Exits
// non-zero on the first failed check; the sanitizers abort on any invalid
// access, leak or undefined operation.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <random>
#include <vector>

#include "stub_launchers.hpp"

using duo::g_stub;

static int g_checks = 0;
#define CHECK(c)                                                            \
  do {                                                                      \
    ++g_checks;                                                             \
    if (!(c)) {                                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);       \
      exit(1);                                                              \
    }                                                                       \
  } while (0)

// Device pointers are never dereferenced on the host: aligned stand-ins.
static void* dev(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x100000000ull + i * 0x10000000ull); }

static duo_layer_desc desc(int B, int Hq, int Hkv, int D, int Hr, int64_t cap,
                           duo_dtype kv = DUO_BF16, duo_dtype rd = DUO_BF16) {
  duo_layer_desc d;
  memset(&d, 0, sizeof(d));
  d.batch = B;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = D;
  d.n_retrieval_kv_heads = Hr;
  d.sink = 16;
  d.recent = 64;
  d.retrieval_capacity = cap;
  d.kv_dtype = kv;
  d.retrieval_dtype = rd;
  d.softmax_scale = 0.088f;
  return d;
}

static void layouts() {
  duo_layout L;
  duo_layer_desc d = desc(1, 32, 8, 128, 4, 1000);
  CHECK(duo_layer_layout(&d, &L) == DUO_OK);
  CHECK(L.v_offset == (size_t)4 * 1000 * 128 * 2);
  CHECK(L.streaming_bytes == (size_t)2 * 4 * 80 * 128 * 2);
  CHECK(duo_layer_layout(nullptr, &L) == DUO_ERR_INVALID_ARG);
  CHECK(duo_layer_layout(&d, nullptr) == DUO_ERR_INVALID_ARG);
  duo_layer_desc bad = d;
  bad.head_dim = 96;
  CHECK(duo_layer_layout(&bad, &L) == DUO_ERR_UNSUPPORTED);
  bad = d;
  bad.n_q_heads = 30;
  CHECK(duo_layer_layout(&bad, &L) == DUO_ERR_INVALID_ARG);
  bad = d;
  bad.batch = 65536;
  CHECK(duo_layer_layout(&bad, &L) == DUO_ERR_UNSUPPORTED);
  bad = desc(65535, 65535, 65535, 128, 1, 1 << 22);
  CHECK(duo_layer_layout(&bad, &L) == DUO_ERR_CAPACITY);
  duo_layer_desc d4 = desc(2, 32, 8, 128, 4, 1 << 20, DUO_FP16, DUO_INT4_G32);
  CHECK(duo_layer_layout(&d4, &L) == DUO_OK);
  CHECK(L.retrieval_bytes == (size_t)2 * 160 * 4 * (1 << 20));
  // every offset is 256-byte aligned
  for (size_t off : {L.v_offset, L.k_sz_offset, L.v_sz_offset, L.ring_v_offset})
    CHECK(off % 256 == 0);
}

static void token_counts_and_failures() {
  duo_layer_desc d = desc(1, 8, 8, 64, 2, 100);
  duo_layer* L = nullptr;
  g_stub.reset();
  CHECK(duo_layer_init(&L, &d, dev(1), dev(2), dev(3), 0, nullptr) == DUO_OK);
  CHECK(g_stub.calls[duo::kZero] == 1 && g_stub.zero_bytes > 0);
  CHECK(duo_append_kv(L, dev(4), dev(5), 60, nullptr) == DUO_OK);
  CHECK(duo_layer_tokens(L) == 60 && g_stub.last_T == 60);
  CHECK(duo_prefill_chunk(L, dev(6), dev(4), dev(5), 30, dev(7), nullptr) == DUO_OK);
  CHECK(duo_layer_tokens(L) == 90);
  CHECK(duo_decode(L, dev(6), dev(4), dev(5), dev(7), nullptr) == DUO_OK);
  CHECK(duo_layer_tokens(L) == 91);
  // capacity: nothing launched, nothing advanced
  const int before = g_stub.calls[duo::kAppendCache];
  CHECK(duo_append_kv(L, dev(4), dev(5), 10, nullptr) == DUO_ERR_CAPACITY);
  CHECK(g_stub.calls[duo::kAppendCache] == before && duo_layer_tokens(L) == 91);
  // misaligned and null arguments
  CHECK(duo_append_kv(L, (char*)dev(4) + 8, dev(5), 1, nullptr) == DUO_ERR_LAYOUT);
  CHECK(duo_decode(L, nullptr, dev(4), dev(5), dev(7), nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(duo_append_kv(L, dev(4), dev(5), 0, nullptr) == DUO_ERR_INVALID_ARG);
  // a failed launch: DUO_ERR_HIP, the count is not advanced
  g_stub.fail_on = duo::kAppendRing;
  CHECK(duo_append_kv(L, dev(4), dev(5), 2, nullptr) == DUO_ERR_HIP);
  CHECK(duo_layer_tokens(L) == 91);
  g_stub.fail_on = duo::kDecode;
  CHECK(duo_decode(L, dev(6), dev(4), dev(5), dev(7), nullptr) == DUO_ERR_HIP);
  CHECK(duo_layer_tokens(L) == 91);
  g_stub.fail_on = -1;
  CHECK(duo_layer_destroy(L) == DUO_OK);
  CHECK(duo_layer_destroy(nullptr) == DUO_OK);
  CHECK(duo_layer_tokens(nullptr) == -1);
  // fp16 and 4-bit layers prefill like bf16 ones: the cache append, both
  // attention launches and the ring append, then the count advances
  const duo_dtype forms[3][2] = {{DUO_FP16, DUO_FP16}, {DUO_FP16, DUO_INT4_G32},
                                 {DUO_BF16, DUO_INT4_G32}};
  for (const auto& f : forms) {
    duo_layer_desc dq = desc(1, 8, 8, 64, 2, 100, f[0], f[1]);
    CHECK(duo_layer_init(&L, &dq, dev(1), dev(2), dev(3), 0, nullptr) == DUO_OK);
    g_stub.reset();
    CHECK(duo_prefill_chunk(L, dev(6), dev(4), dev(5), 3, dev(7), nullptr) == DUO_OK);
    CHECK(g_stub.calls[duo::kAppendCache] == 1 && g_stub.calls[duo::kPrefillRetrieval] == 1 &&
          g_stub.calls[duo::kPrefillStreaming] == 1 && g_stub.calls[duo::kAppendRing] == 1);
    CHECK(duo_layer_tokens(L) == 3);
    CHECK(duo_prefill_chunk(L, dev(6), dev(4), dev(5), 98, dev(7), nullptr) == DUO_ERR_CAPACITY);
    CHECK(duo_layer_tokens(L) == 3);
    duo_layer_destroy(L);
  }
  g_stub.reset();
  // init validation
  CHECK(duo_layer_init(&L, &d, dev(1), dev(2), nullptr, 0, nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(duo_layer_init(&L, &d, (char*)dev(1) + 16, dev(2), dev(3), 0, nullptr) == DUO_ERR_LAYOUT);
  CHECK(duo_layer_init(&L, &d, dev(1), dev(2), dev(3), 101, nullptr) == DUO_ERR_CAPACITY);
}

// 70 ragged sequences decode in slices of 64 and 6, then batch-wide once they
// hold equal counts: every launch must find the split-K counters and
// partials at the same workspace offsets, and each slice its own cache rows.
static void ragged_views(duo_dtype kv, duo_dtype rd) {
  const int B = 70;
  duo_layer_desc d = desc(B, 16, 16, 128, 8, 400, kv, rd);
  std::vector<int64_t> n0(B);
  for (int b = 0; b < B; ++b) n0[b] = 1 + (b * 37) % 150;
  duo_layer* L = nullptr;
  g_stub.reset();
  CHECK(duo_layer_init_ragged(&L, &d, dev(1), dev(2), dev(3), n0.data(), nullptr) == DUO_OK);
  CHECK(duo_layer_tokens(L) == *std::max_element(n0.begin(), n0.end()));
  CHECK(duo_append_kv(L, dev(4), dev(5), 1, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(duo_decode(L, dev(6), dev(4), dev(5), dev(7), nullptr) == DUO_OK);
  CHECK(g_stub.decodes.size() == 2);
  const duo::DecodeLaunch s0 = g_stub.decodes[0], s1 = g_stub.decodes[1];
  CHECK(s0.batch == 64 && s1.batch == 6);
  CHECK(s0.counters == s1.counters && s0.ml == s1.ml && s0.acc == s1.acc);
  duo_layout lay;
  CHECK(duo_layer_layout(&d, &lay) == DUO_OK);
  const size_t per_seq = rd == DUO_INT4_G32 ? (size_t)8 * 416 * 64 : (size_t)8 * 400 * 128 * 2;
  CHECK(s1.rbuf_k - s0.rbuf_k == (ptrdiff_t)(64 * per_seq));
  for (int b = 0; b < B; ++b) CHECK(duo_layer_sequence_tokens(L, b) == n0[b] + 1);
  // catch up to equal counts one sequence at a time
  const int64_t top = 200;
  for (int b = 0; b < B; ++b) {
    const int64_t have = duo_layer_sequence_tokens(L, b);
    CHECK(duo_append_kv_seq(L, b, dev(4), dev(5), (int)(top - have), nullptr) == DUO_OK);
  }
  CHECK(duo_append_kv_seq(L, B, dev(4), dev(5), 1, nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(duo_append_kv_seq(L, 0, dev(4), dev(5), 1000, nullptr) == DUO_ERR_CAPACITY);
  g_stub.decodes.clear();
  CHECK(duo_decode(L, dev(6), dev(4), dev(5), dev(7), nullptr) == DUO_OK);
  CHECK(g_stub.decodes.size() == 1 && g_stub.decodes[0].batch == B && !g_stub.decodes[0].ragged);
  CHECK(g_stub.decodes[0].counters == s0.counters && g_stub.decodes[0].ml == s0.ml &&
        g_stub.decodes[0].acc == s0.acc);
  CHECK(duo_layer_tokens(L) == top + 1);
  CHECK(duo_layer_sequence_tokens(L, -1) == -1 && duo_layer_sequence_tokens(L, B) == -1);
  duo_layer_destroy(L);
}

static void stateless_calls() {
  duo_layer_desc d = desc(1, 32, 32, 128, 0, 0);
  float* a = (float*)dev(9);
  CHECK(duo_mixed_forward(&d, dev(1), dev(2), dev(3), a, 100, dev(4), nullptr) == DUO_OK);
  CHECK(duo_mixed_forward(&d, dev(1), dev(2), dev(3), a, 0, dev(4), nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(duo_mixed_forward_block(&d, dev(1), dev(2), dev(3), a, 100, 32, dev(4), nullptr) ==
        DUO_ERR_UNSUPPORTED);
  const size_t ws = duo_mixed_alpha_grad_workspace(&d, 16384);
  CHECK(ws == (size_t)32 * 64 * 4);
  CHECK(duo_mixed_alpha_grad(&d, dev(1), dev(2), dev(3), dev(5), a, 0.05f, 16384, a, dev(6), ws,
                             nullptr) == DUO_OK);
  CHECK(duo_mixed_alpha_grad(&d, dev(1), dev(2), dev(3), dev(5), a, 0.05f, 16384, a, dev(6),
                             ws - 4, nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(duo_mixed_alpha_grad_noalloc(&d, dev(1), dev(2), dev(3), dev(5), a, 0.05f, 16384, 0, a,
                                     nullptr) == DUO_OK);
  CHECK(g_stub.grad_partial != nullptr);
  duo_layer_desc big = desc(64, 32, 32, 128, 0, 0);
  CHECK(duo_mixed_alpha_grad_noalloc(&big, dev(1), dev(2), dev(3), dev(5), a, 0.05f, 8193, 0, a,
                                     nullptr) == DUO_ERR_CAPACITY);
}

static void host_helpers() {
  std::mt19937 rng(1234);
  for (int n = 1; n <= 40; ++n) {
    std::vector<uint8_t> mask(n);
    for (auto& m : mask) m = rng() % 2;
    std::vector<int32_t> perm(n);
    int32_t nr = -1;
    CHECK(duo_head_permutation(mask.data(), n, perm.data(), &nr) == DUO_OK);
    CHECK(nr == std::count(mask.begin(), mask.end(), 1));
    std::vector<int32_t> sorted = perm;
    std::sort(sorted.begin(), sorted.end());
    for (int i = 0; i < n; ++i) CHECK(sorted[i] == i);
    for (int i = 0; i < n; ++i) CHECK((mask[perm[i]] != 0) == (i < nr));
    // gates: the floor(sparsity * n) smallest become streaming heads
    std::vector<float> alpha(n);
    for (auto& x : alpha) x = (float)(rng() % 1000) / 1000.0f;
    std::vector<uint8_t> out(n);
    CHECK(duo_binarize_gates(alpha.data(), n, 0.5, out.data()) == DUO_OK);
    const int k = (int)(0.5 * n);
    std::vector<float> s = alpha;
    std::sort(s.begin(), s.end());
    const float tau = k < n ? s[k] : 0.0f;
    for (int i = 0; i < n; ++i) CHECK(out[i] == (k < n && alpha[i] >= tau ? 1 : 0));
    CHECK(duo_binarize_gates(alpha.data(), n, 1.5, out.data()) == DUO_ERR_INVALID_ARG);
    // weight reorder and its inverse
    const int rows = 3, row_bytes = 7;
    std::vector<uint8_t> w((size_t)n * rows * row_bytes), r1(w.size()), r2(w.size());
    for (auto& x : w) x = (uint8_t)rng();
    CHECK(duo_reorder_head_rows(w.data(), r1.data(), perm.data(), n, rows, row_bytes) == DUO_OK);
    std::vector<int32_t> inv(n);
    for (int i = 0; i < n; ++i) inv[perm[i]] = i;
    CHECK(duo_reorder_head_rows(r1.data(), r2.data(), inv.data(), n, rows, row_bytes) == DUO_OK);
    CHECK(w == r2);
    CHECK(duo_reorder_head_rows(w.data(), w.data(), perm.data(), n, rows, row_bytes) ==
          DUO_ERR_LAYOUT);
    if (n > 1) {
      std::vector<int32_t> dup = perm;
      dup[0] = dup[1];
      CHECK(duo_reorder_head_rows(w.data(), r1.data(), dup.data(), n, rows, row_bytes) ==
            DUO_ERR_INVALID_ARG);
    }
  }
  for (int64_t p = 0; p < 300; ++p) {
    const int32_t s = duo_ring_slot(p, 16, 64);
    CHECK(s == (p < 16 ? p : 16 + (p - 16) % 64));
  }
  CHECK(duo_ring_slot(-1, 16, 64) == -1 && duo_ring_slot(0, 16, 0) == -1);
  for (int st = 0; st <= 6; ++st) CHECK(duo_status_string((duo_status)st) != nullptr);
}

int main() {
  layouts();
  token_counts_and_failures();
  ragged_views(DUO_BF16, DUO_BF16);
  ragged_views(DUO_FP16, DUO_INT4_G32);
  stateless_calls();
  host_helpers();
  printf("host ABI checks passed: %d\n", g_checks);
  return 0;
}
