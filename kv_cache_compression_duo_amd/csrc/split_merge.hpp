// Log-sum-exp merge of split-K partial softmax states, run by the last block
// of a (batch, KV head) to finish. A split s holds (m_s, l_s, a_s[D]) with
// scores in the log2 domain: m_s = max score, l_s = sum 2^(score - m_s),
// a_s = sum 2^(score - m_s) v. The merged output is
//   o = sum_s 2^(m_s - M) a_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s.
// All threads of the block take part. Partials are read with agent-scope
// loads, which see the other blocks' agent-scope stores without a cache
// invalidate.
#pragma once
#include "device_common.hpp"

namespace duo {

// Scratch of a merge by a block of NT threads.
template <int NT>
struct MergeLds {
  float w[2 * NT];
  float part[NT];
};

__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 ld_agent2(const float* p) {  // 8-byte aligned
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// ml: [G][max_split][2], acc: [G][max_split][D]; out row g at out + g*D (bf16).
// Thread (part, d) folds the splits part, part + P, ... into a running
// (m, l, o). D is a multiple of 64, so `part` is uniform in a wave and the
// split indices and addresses are scalar. Loads are issued UN splits at a
// time with clamped (always valid) indices, so a batch costs one memory round
// trip; entries past the last split get weight 0. The P parts of each channel
// are then folded in LDS.
template <int D, int G, int NT>
__device__ void merge_splits(MergeLds<NT>& s, const float* __restrict__ ml,
                             const float* __restrict__ acc, int max_split, int n_split,
                             uint16_t* __restrict__ out) {
  constexpr int P = NT / D;  // threads per output channel
  constexpr int UN = 16;
  static_assert(D % 64 == 0, "a wave must not straddle two parts");
  const int t = threadIdx.x;
  const int d = t % D;
  const int part = __builtin_amdgcn_readfirstlane(t / D);
  for (int g = 0; g < G; ++g) {
    const float* mlg = ml + (int64_t)g * max_split * 2;
    const float* ag = acc + (int64_t)g * max_split * D + d;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    for (int sp0 = part; sp0 < n_split; sp0 += UN * P) {
      float2 mlv[UN];
      float aa[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int sp = sp0 + u * P < n_split ? sp0 + u * P : n_split - 1;
        mlv[u] = ld_agent2(mlg + sp * 2);
        aa[u] = ld_agent(ag + (int64_t)sp * D);
      }
      float mx = m;
#pragma unroll
      for (int u = 0; u < UN; ++u) mx = fmaxf(mx, mlv[u].x);
      // a split with no row (m = -inf: past a shorter sequence's end) has
      // weight 0; guard -inf - -inf when every split so far is empty
      const float c = m == -INFINITY ? 0.0f : fast_exp2(m - mx);
      l *= c;
      o *= c;
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const bool use = sp0 + u * P < n_split && mlv[u].x != -INFINITY;
        const float w = use ? fast_exp2(mlv[u].x - mx) : 0.0f;
        l = fmaf(mlv[u].y, w, l);
        o = fmaf(aa[u], w, o);
      }
      m = mx;
    }
    s.part[t] = m;
    s.w[t] = l;
    s.w[NT + t] = o;
    __syncthreads();
    if (t < D) {
      float M = s.part[t];
#pragma unroll
      for (int p = 1; p < P; ++p) M = fmaxf(M, s.part[p * D + t]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const float mp = s.part[p * D + t];
        const float w = mp == -INFINITY ? 0.0f : fast_exp2(mp - M);
        L = fmaf(s.w[p * D + t], w, L);
        O = fmaf(s.w[NT + p * D + t], w, O);
      }
      out[(int64_t)g * D + t] = (uint16_t)f2bf(O / L);
    }
    __syncthreads();
  }
}

}  // namespace duo
