// Host-only stand-ins for the kernel launchers of the C-ABI library, so that
// its front end (descriptor validation, layout arithmetic, token counts,
// ragged views, host helpers) can be built with AddressSanitizer and driven
// without a GPU. Each launcher records what it was given and succeeds, unless
// a test asks it to fail.
#include "stub_launchers.hpp"

namespace duo {

StubLog g_stub;

static hipError_t result(int which) {
  ++g_stub.calls[which];
  return g_stub.fail_on == which ? hipErrorLaunchFailure : hipSuccess;
}

hipError_t launch_zero(void*, size_t bytes, hipStream_t) {
  g_stub.zero_bytes = bytes;
  return result(kZero);
}
hipError_t launch_append_cache(const duo_layer* L, const void*, const void*, int T, hipStream_t) {
  g_stub.last_T = T;
  g_stub.last_n = L->n;
  return result(kAppendCache);
}
hipError_t launch_append_ring(const duo_layer* L, const void*, const void*, int T, hipStream_t) {
  g_stub.last_T = T;
  g_stub.last_n = L->n;
  return result(kAppendRing);
}
static hipError_t record_decode(const duo_layer* L, int which) {
  const WsView ws = ws_view(L);
  DecodeLaunch d;
  d.batch = L->d.batch;
  d.n = L->n;
  d.ragged = L->ragged;
  d.counters = ws.counters;
  d.ml = ws.ml;
  d.acc = ws.acc;
  d.rbuf_k = L->rbuf + L->lay.k_offset;
  g_stub.decodes.push_back(d);
  return result(which);
}
hipError_t launch_decode(const duo_layer* L, const void*, const void*, const void*, void*,
                         hipStream_t) {
  return record_decode(L, kDecode);
}
hipError_t launch_decode_int4(const duo_layer* L, const void*, const void*, const void*, void*,
                              hipStream_t) {
  return record_decode(L, kDecodeInt4);
}
hipError_t launch_prefill_retrieval(const duo_layer* L, const void*, int T, void*, hipStream_t) {
  g_stub.last_T = T;
  g_stub.last_n = L->n;
  return result(kPrefillRetrieval);
}
hipError_t launch_prefill_streaming(const duo_layer* L, const void*, const void*, const void*,
                                    int T, void*, hipStream_t) {
  g_stub.last_T = T;
  g_stub.last_n = L->n;
  return result(kPrefillStreaming);
}
hipError_t launch_mixed(const duo_layer_desc&, const void*, const void*, const void*,
                        const float*, int T, int, void*, hipStream_t) {
  g_stub.last_T = T;
  return result(kMixed);
}
hipError_t launch_mixed_alpha_grad(const duo_layer_desc&, const void*, const void*, const void*,
                                   const void*, const float*, float, int T, int, float*,
                                   float* partial, hipStream_t) {
  g_stub.last_T = T;
  g_stub.grad_partial = partial;
  return result(kMixedGrad);
}
static float g_fake_scratch[16];
hipError_t grad_scratch(float** out) {
  *out = g_fake_scratch;
  return hipSuccess;
}

}  // namespace duo

// The two runtime queries the front end makes (device and compute-unit
// count), answered as one MI355X would, so no HIP runtime is linked.
extern "C" hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}
