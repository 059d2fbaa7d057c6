// Fused decode step for bf16/fp16 caches: append of the new token, split-K
// attention of retrieval heads over the full cache, attention of streaming
// heads over the sink + recent ring, and the log-sum-exp merge of split-K
// partials -- one launch per step.
//
// What is computed follows the xllm-io review "DuoAttention: Efficient
// Long-Context LLM Inference with Retrieval and Streaming Heads", section 三:
// 推理流程 (two caches per layer, new Q/K/V split along heads, outputs
// concatenated along heads) and 核心公式 (full softmax attention for retrieval
// heads, Lambda-masked attention for streaming heads). Splitting the key range
// and merging partial softmax states is the split-K decoding idea the
// paperlayer summary lists among complementary system optimisations (section
// 4, FlashDecoding); the partials here are merged by the last block to finish.
//
// Design for gfx950: decode is bound by HBM reads of the retrieval cache. A
// wave streams 32 cache rows per tile with 16-byte loads (D/8 lanes per row,
// rows contiguous in memory), K and V loads of a tile are issued together, and
// the G query heads of a KV head share every K/V load. Scores are reduced
// across the lanes of a row with DPP; only the tile maximum crosses rows.
// Blocks [0, Hs) are streaming heads, the next Hr*n_split blocks are
// retrieval splits, sized so that the grid fills the resident block slots of
// the chip once. The new token is read from the input (never from the
// cache) in this launch, and written to its cache row / ring slot by one
// block, so no block reads memory another block writes.
#include <stdlib.h>

#include "device_common.hpp"
#include "duo_internal.hpp"
#include "split_merge.hpp"

namespace duo {

struct DecodeArgs {
  const uint16_t* q;      // [B][Hq][D] bf16
  const uint16_t* k_new;  // [B][Hkv][D]
  const uint16_t* v_new;
  uint16_t* out;          // [B][Hq][D] bf16
  uint16_t* kc;           // [B][Hr][cap][D]
  uint16_t* vc;
  uint16_t* kr;           // [B][Hs][W][D]
  uint16_t* vr;
  uint32_t* counters;     // [B][Hr]
  float* ml;              // [B][Hr][G][max_split][2]
  float* acc;             // [B][Hr][G][max_split][D]
  int Hq, Hkv, Hr, Hs, S, R, max_split;
  int64_t cap;
  int n;                  // position of the new token
  int n_split, split_tokens;
  float qscale;           // softmax scale * log2(e)
};

constexpr int kWaves = 4;
constexpr int kTile = 32;  // rows per wave-tile

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
template <int D, int G, typename Tag, typename KPtr, typename VPtr>
__device__ __forceinline__ void attend_rows(WaveState<G>& st, const float (&qf)[G][8], int r0,
                                            int r1, KPtr kptr, VPtr vptr) {
  constexpr int LPR = D / 8;       // lanes per row
  constexpr int RPL = 64 / LPR;    // rows per load
  constexpr int U = kTile / RPL;   // loads per tile
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  constexpr int stride = kWaves * kTile;
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

// Merge the waves' states through LDS. On return, thread t < G*D/8... holds
// nothing; the merged (m, l, acc[D]) per head is left in LDS `red`.
template <int D, int G>
struct BlockRed {
  float m[kWaves][G], l[kWaves][G], acc[kWaves][G][D];
  float M[G], L[G];
};

template <int D, int G>
__device__ __forceinline__ void block_merge(BlockRed<D, G>& red, const WaveState<G>& st) {
  constexpr int LPR = D / 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  __syncthreads();
  if (threadIdx.x < G) {
    int g = threadIdx.x;
    float M = red.m[0][g];
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red.m[w][g]);
    float Lsum = 0.0f;
    for (int w = 0; w < kWaves; ++w)
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
    for (int w = 0; w < kWaves; ++w)
      if (red.m[w][g] != -INFINITY) a += red.acc[w][g][dd] * fast_exp2(red.m[w][g] - M);
    red.acc[0][g][dd] = a;
  }
  __syncthreads();
}

template <int D, int G, typename Tag>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;
  __shared__ BlockRed<D, G> red;
  __shared__ MergeLds mlds;
  __shared__ int is_last;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int lc = lane % LPR;
  // Streaming heads take the first Hs blocks (dispatched first, short), the
  // retrieval splits the rest.
  const bool retrieval = (int)blockIdx.x >= a.Hs;
  const int rb = (int)blockIdx.x - a.Hs;
  const int kvh = retrieval ? rb / a.n_split : a.Hr + (int)blockIdx.x;

  // query fragments, pre-scaled into the log2 domain
  float qf[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint16_t* qp = a.q + ((int64_t)b * a.Hq + kvh * G + g) * D + lc * 8;
    float t[8];
    unpack8<Bf16Tag>(ld16(qp), t);
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[g][c] = t[c] * a.qscale;
  }
  const uint16_t* knew = a.k_new + ((int64_t)b * a.Hkv + kvh) * D;
  const uint16_t* vnew = a.v_new + ((int64_t)b * a.Hkv + kvh) * D;
  WaveState<G> st;

  if (retrieval) {
    const int split = rb % a.n_split;
    const int r0 = split * a.split_tokens;
    int r1 = r0 + a.split_tokens;
    if (r1 > a.n + 1) r1 = a.n + 1;
    const int64_t hb = (int64_t)b * a.Hr + kvh;
    const uint16_t* kc = a.kc + hb * a.cap * D;
    const uint16_t* vc = a.vc + hb * a.cap * D;
    const int n = a.n;
    auto kp = [=](int row) { return row == n ? knew : kc + (int64_t)row * D; };
    auto vp = [=](int row) { return row == n ? vnew : vc + (int64_t)row * D; };
    attend_rows<D, G, Tag>(st, qf, r0, r1, kp, vp);
    // the new token's cache row (read by no block of this launch)
    if (split == 0 && threadIdx.x < LPR) {
      st16(a.kc + (hb * a.cap + n) * D + threadIdx.x * 8, ld16(knew + threadIdx.x * 8));
      st16(a.vc + (hb * a.cap + n) * D + threadIdx.x * 8, ld16(vnew + threadIdx.x * 8));
    }
    block_merge<D, G>(red, st);
    // Publish this split's partial state. The partials are written and read
    // with agent-scope (cache-coherent) accesses and the writes are drained
    // before the arrival count is bumped, so no cache-wide writeback or
    // invalidate is needed on this path.
    const int64_t pbase = (hb * G) * a.max_split;
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      int g = i / D, dd = i % D;
      __hip_atomic_store(a.acc + (pbase + (int64_t)g * a.max_split + split) * D + dd,
                         red.acc[0][g][dd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x < G) {
      int g = threadIdx.x;
      float* mlp = a.ml + (pbase + (int64_t)g * a.max_split + split) * 2;
      __hip_atomic_store(mlp, red.M[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mlp + 1, red.L[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t prev = __hip_atomic_fetch_add(a.counters + hb, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      is_last = (prev == (uint32_t)(a.n_split - 1));
    }
    __syncthreads();
    if (!is_last) return;
    // last block of this head: merge all splits
    merge_splits<D, G>(mlds, a.ml + pbase * 2, a.acc + pbase * D, a.max_split, a.n_split,
                       a.out + ((int64_t)b * a.Hq + kvh * G) * D);
    if (threadIdx.x == 0)
      __hip_atomic_store(a.counters + hb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // streaming head: ring slots after the append hold exactly the keys the
    // Lambda mask allows for the new token
    const int hs = kvh - a.Hr;
    const int W = a.S + a.R;
    const int nslots = a.n + 1 < W ? a.n + 1 : W;
    const int slot_new = a.n < a.S ? a.n : a.S + (a.n - a.S) % a.R;
    const int64_t hb = (int64_t)b * a.Hs + hs;
    const uint16_t* kr = a.kr + hb * W * D;
    const uint16_t* vr = a.vr + hb * W * D;
    auto kp = [=](int row) { return row == slot_new ? knew : kr + (int64_t)row * D; };
    auto vp = [=](int row) { return row == slot_new ? vnew : vr + (int64_t)row * D; };
    attend_rows<D, G, Tag>(st, qf, 0, nslots, kp, vp);
    if (threadIdx.x < LPR) {
      st16(a.kr + (hb * W + slot_new) * D + threadIdx.x * 8, ld16(knew + threadIdx.x * 8));
      st16(a.vr + (hb * W + slot_new) * D + threadIdx.x * 8, ld16(vnew + threadIdx.x * 8));
    }
    block_merge<D, G>(red, st);
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      int g = i / D, dd = i % D;
      a.out[((int64_t)b * a.Hq + kvh * G + g) * D + dd] =
          (uint16_t)f2bf(red.acc[0][g][dd] / red.L[g]);
    }
  }
}

static int env_split_tokens() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("DUO_DECODE_SPLIT_TOKENS");
    v = e ? atoi(e) : 0;
    if (v < 0) v = 0;
  }
  return v;
}

// Resident 256-thread blocks of a kernel on the current device (all CUs).
template <typename K>
static int resident_blocks(K kernel) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, 256, 0) != hipSuccess ||
      cus <= 0 || per <= 0)
    return 512;
  return cus * per;
}

// Split size: the Hr*B*n_split retrieval blocks plus the Hs*B streaming
// blocks fill the resident slots once (equal-sized splits finish together);
// splits are whole 32-row tiles and at least kMinSplitTokens rows.
template <int D, int G, typename Tag>
static hipError_t launch_t(DecodeArgs a, int B, int64_t rows, int max_split, hipStream_t s) {
  int st = env_split_tokens();
  if (st <= 0 && a.Hr > 0) {
    static int resident = 0;  // per kernel instance
    if (!resident) resident = resident_blocks(decode_kernel<D, G, Tag>);
    int slots = resident / B - a.Hs;
    int per_head = slots / a.Hr;
    if (per_head < 1) per_head = 1;
    int64_t t = (rows + per_head - 1) / per_head;
    st = (int)((t + kTile - 1) / kTile * kTile);
  }
  if (st < kMinSplitTokens) st = kMinSplitTokens;
  a.split_tokens = st;
  a.n_split = a.Hr > 0 ? (int)((rows + st - 1) / st) : 0;
  if (a.n_split > max_split) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.Hr * a.n_split + a.Hs), (unsigned)B);
  decode_kernel<D, G, Tag><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, typename Tag>
static hipError_t launch_g(int G, const DecodeArgs& a, int B, int64_t rows, int max_split,
                           hipStream_t s) {
  switch (G) {
    case 1: return launch_t<D, 1, Tag>(a, B, rows, max_split, s);
    case 2: return launch_t<D, 2, Tag>(a, B, rows, max_split, s);
    case 4: return launch_t<D, 4, Tag>(a, B, rows, max_split, s);
    default: return launch_t<D, 8, Tag>(a, B, rows, max_split, s);
  }
}

hipError_t launch_decode(const duo_layer* L, const void* q, const void* k_new,
                         const void* v_new, void* out, hipStream_t s) {
  const duo_layer_desc& d = L->d;
  DecodeArgs a;
  WsView ws = ws_view(L);
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.out = static_cast<uint16_t*>(out);
  a.kc = reinterpret_cast<uint16_t*>(L->rbuf + L->lay.k_offset);
  a.vc = reinterpret_cast<uint16_t*>(L->rbuf + L->lay.v_offset);
  a.kr = reinterpret_cast<uint16_t*>(L->sbuf + L->lay.ring_k_offset);
  a.vr = reinterpret_cast<uint16_t*>(L->sbuf + L->lay.ring_v_offset);
  a.counters = ws.counters;
  a.ml = ws.ml;
  a.acc = ws.acc;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.Hr = L->Hr;
  a.Hs = L->Hs;
  a.S = d.sink;
  a.R = d.recent;
  a.max_split = L->max_split;
  a.cap = d.retrieval_capacity;
  a.n = (int)L->n;
  a.qscale = d.softmax_scale * kLog2e;
  const int64_t rows = L->n + 1;
  const int B = d.batch;
  if (d.head_dim == 128) {
    if (d.kv_dtype == DUO_FP16) return launch_g<128, Fp16Tag>(L->G, a, B, rows, L->max_split, s);
    return launch_g<128, Bf16Tag>(L->G, a, B, rows, L->max_split, s);
  }
  if (d.kv_dtype == DUO_FP16) return launch_g<64, Fp16Tag>(L->G, a, B, rows, L->max_split, s);
  return launch_g<64, Bf16Tag>(L->G, a, B, rows, L->max_split, s);
}

}  // namespace duo

