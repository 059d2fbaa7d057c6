// Records of the stand-in launchers (see stub_launchers.cpp).
#pragma once
#include <vector>

#include "../../kv_cache_compression_duo_amd/csrc/duo_internal.hpp"

namespace duo {

enum StubKind {
  kZero, kAppendCache, kAppendRing, kDecode, kDecodeInt4, kPrefillRetrieval,
  kPrefillStreaming, kMixed, kMixedGrad, kStubKinds
};

struct DecodeLaunch {
  int batch;
  int64_t n;
  bool ragged;
  const void* counters;
  const void* ml;
  const void* acc;
  const char* rbuf_k;
};

struct StubLog {
  int calls[kStubKinds] = {};
  int fail_on = -1;  // launcher kind that returns an error, or -1
  int last_T = 0;
  int64_t last_n = 0;
  size_t zero_bytes = 0;
  const float* grad_partial = nullptr;
  std::vector<DecodeLaunch> decodes;
  void reset() { *this = StubLog(); }
};

extern StubLog g_stub;

}  // namespace duo
