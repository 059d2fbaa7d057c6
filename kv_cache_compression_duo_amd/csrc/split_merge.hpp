// Publication and log-sum-exp merge of split-K partial softmax states. Every
// split block of a (batch, KV head) publishes its state; the last block to
// arrive merges them. A split s holds (m_s, l_s, a_s[D]) with scores in the
// log2 domain: m_s = max score, l_s = sum 2^(score - m_s),
// a_s = sum 2^(score - m_s) v. The merged output is
//   o = sum_s 2^(m_s - M) a_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s.
// Partials are written and read with device-coherent (agent-scope) accesses,
// so the merging block sees the other blocks' partials without a cache
// writeback or invalidate. They move in 16-byte accesses: a merge issues a
// few loads per thread instead of one per split and channel (its round trip
// is on the critical path of the step).
#pragma once
#include "device_common.hpp"

namespace duo {

// Cache policy of a device-coherent access on this target (SC1: the bits the
// compiler sets for agent-scope atomic loads and stores).
constexpr int kCpolAgent = 16;

__device__ __forceinline__ float4 ld_agent16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  const v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kCpolAgent);
  return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                     __uint_as_float(x.w));
}
__device__ __forceinline__ float2 ld_agent8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  const v2 x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, kCpolAgent);
  return make_float2(__uint_as_float(x.x), __uint_as_float(x.y));
}
__device__ __forceinline__ void st_agent16(__amdgpu_buffer_rsrc_t r, uint32_t voff, float4 v) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  const v4 x = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)voff, 0, kCpolAgent);
}
__device__ __forceinline__ void st_agent8(__amdgpu_buffer_rsrc_t r, uint32_t voff, float2 v) {
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  const v2 x = {__float_as_uint(v.x), __float_as_uint(v.y)};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)voff, 0, kCpolAgent);
}

// The partials of one (batch, KV head): ml [G][max_split][2] and acc
// [G][max_split][D] floats (each below 2^31 bytes, checked on the host).
struct PartialView {
  __amdgpu_buffer_rsrc_t ml, acc;
};
template <int D, int G>
__device__ __forceinline__ PartialView partial_view(float* ml, float* acc, int max_split) {
  PartialView v;
  v.ml = wave_rsrc(ml, (uint32_t)(G * max_split * 2 * 4));
  v.acc = wave_rsrc(acc, (uint32_t)(G * max_split * D * 4));
  return v;
}

// Publish split `split`'s state: acc0 [G][D] (block-shared), M[G], L[G].
// Returns once the stores have completed (the caller then signals arrival).
template <int D, int G>
__device__ __forceinline__ void publish_partial(const PartialView& pv, int max_split, int split,
                                                const float* acc0, const float* M,
                                                const float* L) {
  constexpr int Q = D / 4;
  for (int i = threadIdx.x; i < G * Q; i += blockDim.x) {
    const int g = i / Q, c4 = i % Q;
    const float4 v = *reinterpret_cast<const float4*>(acc0 + g * D + 4 * c4);
    st_agent16(pv.acc, (uint32_t)(((g * max_split + split) * D + 4 * c4) * 4), v);
  }
  if ((int)threadIdx.x < G) {
    const int g = threadIdx.x;
    st_agent8(pv.ml, (uint32_t)((g * max_split + split) * 8), make_float2(M[g], L[g]));
  }
  __builtin_amdgcn_s_waitcnt(0);  // the stores have reached the coherent level
}

// Scratch of a merge by a block of NT threads: a running state per thread.
template <int NT>
struct MergeLds {
  float m[NT], l[NT];
  float4 o[NT];
};

// Merge the n_split partials into out rows g = 0..G-1 at out + g*D (bf16), all
// heads in one pass. Thread (part, g, c4) folds the splits part, part + P, ...
// of head g for channels 4*c4..4*c4+3 (P = NT / (G * D/4) parts): each split
// costs it one 16-byte acc load and one 8-byte (m, l) load, issued UN splits
// at a time with clamped (always valid) indices so that a batch is one memory
// round trip (16 to 64 splits per round trip); entries past
// the last split get weight 0. The P parts of each (head, channel quadruple)
// are then folded through LDS.
template <int D, int G, int NT>
__device__ void merge_splits(MergeLds<NT>& s, const PartialView& pv, int max_split, int n_split,
                             uint16_t* __restrict__ out) {
  constexpr int Q = D / 4;     // 16-byte columns of a partial row
  constexpr int GQ = G * Q;    // (head, column) pairs
  static_assert(NT % GQ == 0, "whole partial rows of every head per pass");
  constexpr int P = NT / GQ;   // splits folded in parallel per pair
  constexpr int UN = P >= 8 ? 4 : (32 / P < 16 ? 32 / P : 16);
  const int t = threadIdx.x;
  const int c4 = t % Q, g = (t / Q) % G, part = t / GQ;
  float m = -INFINITY, l = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int sp0 = part; sp0 < n_split; sp0 += UN * P) {
    float2 mlv[UN];
    float4 av[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int sp = sp0 + u * P < n_split ? sp0 + u * P : n_split - 1;
      const int row = g * max_split + sp;
      mlv[u] = ld_agent8(pv.ml, (uint32_t)(row * 8));
      av[u] = ld_agent16(pv.acc, (uint32_t)((row * D + 4 * c4) * 4));
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < UN; ++u)
      if (sp0 + u * P < n_split) mx = fmaxf(mx, mlv[u].x);
    // a split with no row (m = -inf: past a shorter sequence's end) has
    // weight 0; guard -inf - -inf while every split so far is empty
    const float c = m == -INFINITY ? 0.0f : fast_exp2(m - mx);
    l *= c;
    o.x *= c;
    o.y *= c;
    o.z *= c;
    o.w *= c;
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const bool use = sp0 + u * P < n_split && mlv[u].x != -INFINITY;
      const float w = use ? fast_exp2(mlv[u].x - mx) : 0.0f;
      l = fmaf(mlv[u].y, w, l);
      o.x = fmaf(av[u].x, w, o.x);
      o.y = fmaf(av[u].y, w, o.y);
      o.z = fmaf(av[u].z, w, o.z);
      o.w = fmaf(av[u].w, w, o.w);
    }
    m = mx;
  }
  s.m[t] = m;
  s.l[t] = l;
  s.o[t] = o;
  __syncthreads();
  if (t < GQ) {
    float M = s.m[t];
#pragma unroll
    for (int p = 1; p < P; ++p) M = fmaxf(M, s.m[p * GQ + t]);
    float L = 0.0f;
    float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const float mp = s.m[p * GQ + t];
      const float w = mp == -INFINITY ? 0.0f : fast_exp2(mp - M);
      const float4 op = s.o[p * GQ + t];
      L = fmaf(s.l[p * GQ + t], w, L);
      O.x = fmaf(op.x, w, O.x);
      O.y = fmaf(op.y, w, O.y);
      O.z = fmaf(op.z, w, O.z);
      O.w = fmaf(op.w, w, O.w);
    }
    uint2 pk;
    pk.x = pack_bf16x2(O.x / L, O.y / L);
    pk.y = pack_bf16x2(O.z / L, O.w / L);
    *reinterpret_cast<uint2*>(out + (int64_t)g * D + 4 * c4) = pk;
  }
  __syncthreads();
}

}  // namespace duo
