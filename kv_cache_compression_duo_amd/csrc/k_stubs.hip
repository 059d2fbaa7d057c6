// Temporary: kernels not yet written report an invalid launch.
#include "duo_internal.hpp"
namespace duo {
hipError_t launch_decode_int4(const duo_layer*, const void*, const void*, const void*, void*,
                              hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prefill_retrieval(const duo_layer*, const void*, int, void*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_prefill_streaming(const duo_layer*, const void*, const void*, const void*, int,
                                    void*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mixed(const duo_layer_desc&, const void*, const void*, const void*,
                        const float*, int, void*, hipStream_t) { return hipErrorInvalidValue; }
}
