// Building blocks shared by the decode kernels: per-wave streaming attention
// over rows of a bf16/fp16 KV source (16-byte loads, D/8 lanes per row, G query
// heads per KV head sharing every load) and the merge of the waves' softmax
// states through LDS.
#pragma once
#include "device_common.hpp"

namespace duo {

constexpr int kTile = 16;  // rows per wave-tile

// Per-wave online-softmax state for G query heads over 8 channels per lane.
template <int G>
struct WaveState {
  float m[G], l[G], acc[G][8];
};

// Attend over rows [r0, r1) of a KV source, tiles interleaved across the
// block's waves, with the next tile's K/V loads in flight while the current
// tile is computed. kptr/vptr(row) return the 16-byte-aligned base of a row.
// On return l and acc are summed over the wave's rows (every lane holds the
// totals for its 8 channels); m is the wave's running maximum.
template <int D, int G, typename Tag, int NW, typename KPtr, typename VPtr>
__device__ __forceinline__ void attend_rows(WaveState<G>& st, const float (&qf)[G][8], int r0,
                                            int r1, KPtr kptr, VPtr vptr) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPL = 64 / LPR;    // rows per load
  constexpr int U = kTile / RPL;   // loads per tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lc = lane % LPR, lr = lane / LPR;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[g][c] = 0.0f;
  }
  int t0 = r0 + wave * kTile;
  if (t0 >= r1) return;
  // Loads are unconditional (rows past the range are clamped to the last
  // valid row and masked out of the softmax), so the tile loop is straight-line
  // code and the next tile's loads stay in flight during the current compute.
  auto load = [&](u32x4 (&kb)[U], u32x4 (&vb)[U], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int row = base + u * RPL + lr;
      row = row < r1 ? row : r1 - 1;
      kb[u] = ld16_nt(kptr(row) + lc * 8);
      vb[u] = ld16_nt(vptr(row) + lc * 8);
    }
  };
  auto compute = [&](const u32x4 (&kb)[U], const u32x4 (&vb)[U], int base) {
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8<Tag>(kb[u], kf);
      const int row = base + u * RPL + lr;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) a = fmaf(qf[g][c], kf[c], a);
        a = group_sum<LPR>(a);
        s[u][g] = row < r1 ? a : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float tm = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) tm = fmaxf(tm, s[u][g]);
      if constexpr (LPR == 8) tm = fmaxf(tm, dpp<0x128>(tm));  // row_ror:8 == xor 8
      tm = fmaxf(tm, xor_lane(tm, 16));
      tm = fmaxf(tm, xor_lane(tm, 32));
      const float mn = fmaxf(st.m[g], tm);
      const float corr = fast_exp2(st.m[g] - mn);
      st.m[g] = mn;
      float ls = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] *= corr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(s[u][g] - mn);
        s[u][g] = p;
        ls += p;
      }
      st.l[g] = st.l[g] * corr + ls;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      unpack8<Tag>(vb[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) st.acc[g][c] = fmaf(s[u][g], vf[c], st.acc[g][c]);
    }
  };
  // Ping-pong register buffers; the prefetch is issued even past the end (all
  // rows then clamp to the last valid row, a cached re-read) so that the
  // waits before each compute only cover the tile being computed.
  constexpr int stride = NW * kTile;
  u32x4 ka[U], va[U], kb[U], vb[U];
  load(ka, va, t0);
  for (;;) {
    const int t1 = t0 + stride;
    load(kb, vb, t1);
    compute(ka, va, t0);
    if (t1 >= r1) break;
    t0 = t1 + stride;
    load(ka, va, t0);
    compute(kb, vb, t1);
    if (t0 >= r1) break;
  }
  // Sum l and acc over the row groups of the wave (lanes sharing lc).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (LPR == 8) {
      st.l[g] += dpp<0x128>(st.l[g]);
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] += dpp<0x128>(st.acc[g][c]);
    }
    st.l[g] += xor_lane(st.l[g], 16);
    st.l[g] += xor_lane(st.l[g], 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      st.acc[g][c] += xor_lane(st.acc[g][c], 16);
      st.acc[g][c] += xor_lane(st.acc[g][c], 32);
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Query fragment of a lane: the 8 channels it owns, as raw bf16 pairs (for
// dot products against bf16 keys) and as pre-scaled floats (fp16 keys).
template <int G>
struct QFrag {
  uint32_t w[G][4];
  float f[G][8];
};

// Raw (unscaled for bf16 keys, pre-scaled for fp16 keys) partial dot of the
// lane's 8 channels of query head g with one 16-byte key chunk.
template <typename Tag, int G>
__device__ __forceinline__ float dot8(const QFrag<G>& q, int g, const u32x4& k) {
  float a = 0.0f;
  if constexpr (Tag::is_bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w[g][i]),
                                          __builtin_bit_cast(bf16x2_t, word_of(k, i)), a, false);
  } else {
    float kf[8];
    unpack8<Tag>(k, kf);
#pragma unroll
    for (int c = 0; c < 8; ++c) a = fmaf(q.f[g][c], kf[c], a);
  }
  return a;
}

// Attend over rows [r0, r1) of one head's contiguous cache (D elements per
// row), optionally followed by one extra row (the token being decoded, read
// from its input rather than the cache) handled by wave 0. A wave load covers
// 1 KB = 64 lanes x 16 bytes = RPL consecutive rows, so lane l reads bytes
// [16 l, 16 l + 16) of it from a wave-uniform base and the loads need no
// per-lane arithmetic and no branch (a branch around loads would make the
// compiler drain the prefetch at the join). A tile starts at min(t, r1 - 1)
// and reads kTile rows from there: the cache buffer extends kDecodePadRows rows
// past its last row, so this stays in bounds; rows at or past r1 (any bytes)
// are masked and their values zeroed in the one partial tile of the range.
// Tiles are interleaved across the block's waves with the next tile's loads
// in flight. sscale turns raw dot products into log2-domain scores (softmax
// scale * log2(e) for bf16 keys, 1 for fp16 keys whose query is pre-scaled).
// slab_bytes is the byte range readable from kc (and from vc): the head's
// rows plus the padding, below 2^31. On return l and acc are summed over the
// wave's rows; m is the wave maximum.
template <int D, int G, typename Tag, int NW, int PF = 2>
__device__ __forceinline__ void attend_cache(WaveState<G>& st, const QFrag<G>& q, float sscale,
                                             const uint16_t* __restrict__ kc,
                                             const uint16_t* __restrict__ vc,
                                             uint32_t slab_bytes, int r0, int r1,
                                             const uint16_t* knew, const uint16_t* vnew,
                                             bool with_new) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPL = 64 / LPR;    // rows per load
  constexpr int U = kTile / RPL;   // loads per tile
  constexpr int LOAD = 512;        // elements per wave load (1 KB)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lc = lane % LPR, lr = lane / LPR;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[g][c] = 0.0f;
  }
  // one online-softmax step over the first n_u loads of rows (scores
  // already masked, values of masked rows zeroed)
  auto update = [&](float (&s)[U][G], const u32x4 (&vb)[U], int n_u) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float tm = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u)
        if (u < n_u) tm = fmaxf(tm, s[u][g]);
      if constexpr (LPR == 8) tm = fmaxf(tm, dpp<0x128>(tm));  // row_ror:8 == xor 8
      tm = fmaxf(tm, xor_lane(tm, 16));
      tm = fmaxf(tm, xor_lane(tm, 32));
      // every update holds an allowed row, so mn is finite
      const float mn = fmaxf(st.m[g], tm);
      const float corr = fast_exp2(st.m[g] - mn);
      st.m[g] = mn;
      float ls = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] *= corr;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u < n_u) {
          const float p = fast_exp2(s[u][g] - mn);
          s[u][g] = p;
          ls += p;
        }
      st.l[g] = st.l[g] * corr + ls;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n_u) {
        float vf[8];
        unpack8<Tag>(vb[u], vf);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int c = 0; c < 8; ++c) st.acc[g][c] = fmaf(s[u][g], vf[c], st.acc[g][c]);
      }
  };
  int t0 = r0 + wave * kTile;
  if (t0 < r1) {
    // Buffer loads: the head's rows are one resource (scalar registers), the
    // lane offset is a constant vector register and the row offset a scalar,
    // so no per-tile vector address is built (64-bit address temporaries
    // shared registers with loads in flight and made the loop wait for every
    // outstanding load).
    const __amdgpu_buffer_rsrc_t krs = wave_rsrc(kc, slab_bytes);
    const __amdgpu_buffer_rsrc_t vrs = wave_rsrc(vc, slab_bytes);
    const uint32_t loff = (uint32_t)lane * 16u;
    auto load = [&](u32x4 (&kb)[U], u32x4 (&vb)[U], int t) {
      const int tl = t < r1 ? t : r1 - 1;  // wave-uniform
      const uint32_t soff = (uint32_t)tl * (uint32_t)(D * 2);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kb[u] = buf_ld16_nt(krs, loff, soff + u * LOAD * 2);
        vb[u] = buf_ld16_nt(vrs, loff, soff + u * LOAD * 2);
      }
    };
    auto compute = [&](const u32x4 (&kb)[U], u32x4 (&vb)[U], int t) {
      float s[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) s[u][g] = group_sum<LPR>(dot8<Tag, G>(q, g, kb[u])) * sscale;
      if (t + kTile > r1) {  // the partial tile (wave-uniform)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = t + u * RPL + lr < r1;
#pragma unroll
          for (int g = 0; g < G; ++g) s[u][g] = ok ? s[u][g] : -INFINITY;
          vb[u] = ok ? vb[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
      update(s, vb, U);
    };
    // PF register buffers in a ring: while tile j is computed the loads of
    // tiles j + 1 .. j + PF - 1 are in flight (prefetches past the range
    // clamp to its last row: a cached re-read, never computed)
    constexpr int stride = NW * kTile;
    u32x4 kq[PF][U], vq[PF][U];
#pragma unroll
    for (int p = 0; p + 1 < PF; ++p) load(kq[p], vq[p], t0 + p * stride);
    for (;;) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        load(kq[(p + PF - 1) % PF], vq[(p + PF - 1) % PF], t0 + (p + PF - 1) * stride);
        compute(kq[p], vq[p], t0 + p * stride);
        if (t0 + (p + 1) * stride >= r1) goto tiles_done;  // wave-uniform
      }
      t0 += PF * stride;
    }
  tiles_done:;
  }
  if (with_new && wave == 0) {
    // one more row: lanes of row slot 0 carry it, the others are masked
    float s[U][G];
    u32x4 vb[U];
    const u32x4 k1 = ld16(knew + lc * 8);
    vb[0] = lr == 0 ? ld16(vnew + lc * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float a = group_sum<LPR>(dot8<Tag, G>(q, g, k1)) * sscale;
      s[0][g] = lr == 0 ? a : -INFINITY;
    }
    update(s, vb, 1);
  }
  // Sum l and acc over the row groups of the wave (lanes sharing lc).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (LPR == 8) {
      st.l[g] += dpp<0x128>(st.l[g]);
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] += dpp<0x128>(st.acc[g][c]);
    }
    st.l[g] += xor_lane(st.l[g], 16);
    st.l[g] += xor_lane(st.l[g], 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      st.acc[g][c] += xor_lane(st.acc[g][c], 16);
      st.acc[g][c] += xor_lane(st.acc[g][c], 32);
    }
  }
}

// Merge the waves' states through LDS. On return, thread t < G*D/8... holds
// nothing; the merged (m, l, acc[D]) per head is left in LDS `red`.
template <int D, int G, int NW>
struct alignas(16) BlockRed {
  float acc[NW][G][D];  // first: rows of acc[0] are read as 16-byte vectors
  float m[NW][G], l[NW][G];
  float M[G], L[G];
};

template <int D, int G, int NW>
__device__ __forceinline__ void block_merge_lds(BlockRed<D, G, NW>& red);

template <int D, int G, int NW>
__device__ __forceinline__ void block_merge(BlockRed<D, G, NW>& red, const WaveState<G>& st) {
  constexpr int LPR = D / 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c = 0; c < 8; ++c) red.acc[wave][g][lane * 8 + c] = st.acc[g][c];
      if (lane == 0) {
        red.m[wave][g] = st.m[g];
        red.l[wave][g] = st.l[g];
      }
    }
  }
  block_merge_lds<D, G, NW>(red);
}

// The reduction part of block_merge, for callers that wrote each wave's (m, l,
// acc) into red themselves (m in the log2 domain, -inf for a wave without
// rows).
template <int D, int G, int NW>
__device__ __forceinline__ void block_merge_lds(BlockRed<D, G, NW>& red) {
  __syncthreads();
  if (threadIdx.x < G) {
    int g = threadIdx.x;
    float M = red.m[0][g];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red.m[w][g]);
    float Lsum = 0.0f;
    for (int w = 0; w < NW; ++w)
      Lsum += red.l[w][g] * (red.m[w][g] == -INFINITY ? 0.0f : fast_exp2(red.m[w][g] - M));
    red.M[g] = M;
    red.L[g] = Lsum;
  }
  __syncthreads();
  // merged acc, in place into red.acc[0]
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    int g = i / D, dd = i % D;
    float M = red.M[g];
    float a = 0.0f;
    for (int w = 0; w < NW; ++w)
      if (red.m[w][g] != -INFINITY) a += red.acc[w][g][dd] * fast_exp2(red.m[w][g] - M);
    red.acc[0][g][dd] = a;
  }
  __syncthreads();
}

}  // namespace duo
