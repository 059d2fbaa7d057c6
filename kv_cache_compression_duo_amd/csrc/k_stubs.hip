// Temporary: kernels not yet written report an invalid launch.
#include "duo_internal.hpp"
namespace duo {
hipError_t launch_decode_int4(const duo_layer*, const void*, const void*, const void*, void*,
                              hipStream_t) { return hipErrorInvalidValue; }
}
