// 4-bit group encoding of one token, shared by the cache-append kernel and
// the decode step that quantises its new token in place.
//
// The encoding is this library's reading of the 4-bit KV cache that the
// xllm-io review "DuoAttention: Efficient Long-Context LLM Inference with
// Retrieval and Streaming Heads" names in section 五 量化组合: per token, head
// and 32-channel group, fp16 scale s = (max - min) / 15 and fp16 zero-point
// z = min, codes rint((x - z) / s) clamped to [0, 15] (0 when s == 0), all in
// fp32 with IEEE division so that the codes are reproducible bit for bit;
// the dequantised value is fma(c, s, z) in fp32.
#pragma once
#include "device_common.hpp"

namespace duo {

template <typename Tag>
__device__ __forceinline__ void encode_group_part(const u32x4& raw, uint32_t* codes_out,
                                                  uint32_t* sz_out) {
  // Four consecutive lanes hold one 32-channel group, 8 channels each.
  float x[8];
  unpack8<Tag>(raw, x);
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, x[j]);
    mx = fmaxf(mx, x[j]);
  }
  // min / max over the 4 lanes of the group (quad_perm butterflies)
  mn = fminf(mn, dpp<0xB1>(mn));
  mx = fmaxf(mx, dpp<0xB1>(mx));
  mn = fminf(mn, dpp<0x4E>(mn));
  mx = fmaxf(mx, dpp<0x4E>(mx));
  _Float16 s16 = (_Float16)__fdiv_rn(mx - mn, 15.0f);
  _Float16 z16 = (_Float16)mn;
  float s = (float)s16, z = (float)z16;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float c = 0.0f;
    if (s != 0.0f) {
      c = rintf(__fdiv_rn(x[j] - z, s));
      c = fminf(fmaxf(c, 0.0f), 15.0f);
    }
    packed |= ((uint32_t)c & 0xFu) << (4 * j);
  }
  *codes_out = packed;
  *sz_out = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
            ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
}

// fp32 value of channel j of a lane's 8-channel chunk: fma(c, s, z)
__device__ __forceinline__ float decode_code(uint32_t codes, uint32_t sz, int j) {
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
  const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz >> 16));
  return fmaf((float)((codes >> (4 * j)) & 0xFu), s, z);
}

}  // namespace duo
