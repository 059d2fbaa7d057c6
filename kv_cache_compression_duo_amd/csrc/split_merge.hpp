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

constexpr int kMergeThreads = 256;

struct MergeLds {
  float w[2 * kMergeThreads];
  float part[kMergeThreads];
};

__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ml: [G][max_split][2], acc: [G][max_split][D]; out row g at out + g*D (bf16).
// One pass: thread (part, d) folds the splits part, part+P, ... into a running
// (m, l, o) with independent loads (no dependent round trips through LDS),
// then the P parts of each channel are folded through LDS.
template <int D, int G>
__device__ void merge_splits(MergeLds& s, const float* __restrict__ ml,
                             const float* __restrict__ acc, int max_split, int n_split,
                             uint16_t* __restrict__ out) {
  constexpr int P = kMergeThreads / D;  // threads per output channel
  constexpr int UN = 4;
  const int t = threadIdx.x;
  const int d = t % D, part = t / D;
  for (int g = 0; g < G; ++g) {
    const float* mlg = ml + (int64_t)g * max_split * 2;
    const float* ag = acc + (int64_t)g * max_split * D + d;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    int sp = part;
    for (; sp + (UN - 1) * P < n_split; sp += UN * P) {
      float mm[UN], ll[UN], aa[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        mm[u] = ld_agent(mlg + (sp + u * P) * 2);
        ll[u] = ld_agent(mlg + (sp + u * P) * 2 + 1);
        aa[u] = ld_agent(ag + (int64_t)(sp + u * P) * D);
      }
      float mx = m;
#pragma unroll
      for (int u = 0; u < UN; ++u) mx = fmaxf(mx, mm[u]);
      const float c = fast_exp2(m - mx);
      l *= c;
      o *= c;
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const float w = fast_exp2(mm[u] - mx);
        l = fmaf(ll[u], w, l);
        o = fmaf(aa[u], w, o);
      }
      m = mx;
    }
    for (; sp < n_split; sp += P) {
      const float mi = ld_agent(mlg + sp * 2), li = ld_agent(mlg + sp * 2 + 1);
      const float ai = ld_agent(ag + (int64_t)sp * D);
      const float mx = fmaxf(m, mi);
      const float c = fast_exp2(m - mx), w = fast_exp2(mi - mx);
      l = l * c + li * w;
      o = o * c + ai * w;
      m = mx;
    }
    s.part[t] = m;
    s.w[t] = l;
    s.w[kMergeThreads + t] = o;
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
        O = fmaf(s.w[kMergeThreads + p * D + t], w, O);
      }
      out[(int64_t)g * D + t] = (uint16_t)f2bf(O / L);
    }
    __syncthreads();
  }
}

}  // namespace duo
