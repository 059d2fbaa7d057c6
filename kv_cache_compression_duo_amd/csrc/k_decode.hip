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
// wave streams 16 cache rows per tile with 16-byte loads (D/8 lanes per row,
// rows contiguous in memory), K and V loads of a tile are issued together, and
// the G query heads of a KV head share every K/V load. Scores are reduced
// across the lanes of a row with DPP; only the tile maximum crosses rows.
// Blocks [0, Hs) are streaming heads, the next Hr*n_split blocks are
// retrieval splits, sized to about one block per compute unit. The new token is read from the input (never from the
// cache) in this launch, and written to its cache row / ring slot by one
// block, so no block reads memory another block writes.
#include "device_common.hpp"
#include "decode_common.hpp"
#include "decode_mma.hpp"
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
  uint32_t* counters;     // arrival counts [B][Hr]
  float* ml;              // [B][Hr][G][max_split][2]
  float* acc;             // [B][Hr][G][max_split][D]
  int Hq, Hkv, Hr, Hs, S, R, max_split;
  int64_t cap;
  int n;                  // position of the new token (every sequence unless ragged)
  int n_split, split_tokens;
  int ragged;             // sequences hold different counts (use nseq)
  float qscale;           // softmax scale * log2(e)
  // per-sequence positions last: the fields every block reads stay on
  // the first lines of the argument block
  int nseq[kMaxRaggedBatch];  // position of the new token per sequence
};

// Retrieval heads of layers with four or more query heads per KV head attend
// on the matrix cores (decode_mma.hpp): on the VALU the G dot products and
// accumulations per row made that loop arithmetic-bound. One or two heads
// per KV head keep the VALU loop, which streams at the HBM rate.
template <int G>
constexpr bool decode_on_mfma() { return G >= 4; }
// Waves per block and tiles per wave held in registers (VALU loop): 4 waves
// with 2 tiles of 16 rows (measured on the Llama-2 layer: 8 or 16 waves per
// block, or 3 or 4 tiles in flight per wave, were slower). The matrix-core
// path keeps 4 waves too: each holds two 32-row K/V stages in LDS.
constexpr int kDecodeWaves = 4;
constexpr int kDecodePrefetch = 2;

template <int D, int G, typename Tag>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;
  constexpr int NW = kDecodeWaves;
  constexpr int PF = kDecodePrefetch;
  constexpr bool kMma = decode_on_mfma<G>();
  __shared__ BlockRed<D, G, NW> red;
  // the matrix-core path's per-wave stages (four arrays, so the compiler's
  // tracking of the direct loads tells the stage read from the stage filled)
  constexpr int MS = kMma ? NW * kMmaRows * D : 8;
  __shared__ __align__(16) uint16_t mk0[MS], mk1[MS], mv0[MS], mv1[MS];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int lc = lane % LPR;
  // Streaming heads take the first Hs blocks (dispatched first, short), the
  // retrieval splits the rest.
  const bool retrieval = (int)blockIdx.x >= a.Hs;
  const int rb = (int)blockIdx.x - a.Hs;
  const int kvh = retrieval ? rb / a.n_split : a.Hr + (int)blockIdx.x;
  // this sequence's new-token position (sequences may hold different counts;
  // the splits cover the longest, so a shorter one's last splits are empty)
  int n = a.n;
  if (a.ragged) n = a.nseq[b];  // only layers of at most kMaxRaggedBatch sequences

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
    if (r1 > n + 1) r1 = n + 1;
    const int64_t hb = (int64_t)b * a.Hr + kvh;
    const uint16_t* kc = a.kc + hb * a.cap * D;
    const uint16_t* vc = a.vc + hb * a.cap * D;
    // cache rows [r0, min(r1, n)); the split holding position n adds the
    // new token from its input; splits past n are empty (m = -inf)
    const bool has_new = r0 <= n && r1 == n + 1;
    const uint32_t slab_bytes = (uint32_t)((a.cap + kDecodePadRows) * D * 2);
    if constexpr (kMma) {
      const int wo = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kMmaRows * D;
      attend_cache_mma<D, G, Tag, NW>(red, a.q + ((int64_t)b * a.Hq + kvh * G) * D, a.qscale, kc,
                                      vc, r0, has_new ? n : r1, knew, vnew, has_new,
                                      mk0 + wo, mk1 + wo, mv0 + wo, mv1 + wo);
    } else {
      QFrag<G> qfrag;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4 raw = ld16(a.q + ((int64_t)b * a.Hq + kvh * G + g) * D + lc * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) qfrag.w[g][i] = word_of(raw, i);
#pragma unroll
        for (int c = 0; c < 8; ++c) qfrag.f[g][c] = qf[g][c];
      }
      attend_cache<D, G, Tag, NW, PF>(st, qfrag, Tag::is_bf16 ? a.qscale : 1.0f, kc, vc,
                                      slab_bytes, r0, has_new ? n : r1, knew, vnew, has_new);
    }
    // the new token's cache row (read by no block of this launch)
    if (split == 0 && threadIdx.x < LPR) {
      st16(a.kc + (hb * a.cap + n) * D + threadIdx.x * 8, ld16(knew + threadIdx.x * 8));
      st16(a.vc + (hb * a.cap + n) * D + threadIdx.x * 8, ld16(vnew + threadIdx.x * 8));
    }
    if constexpr (kMma)
      block_merge_lds<D, G, NW>(red);
    else
      block_merge<D, G, NW>(red, st);
    // Publish this split's partial state. The partials are written and read
    // with device-coherent accesses and the writes complete before the arrival
    // count is bumped, so no cache-wide writeback or invalidate is needed on
    // this path; the last block of the head to arrive merges.
    const int64_t pbase = (hb * G) * a.max_split;
    const PartialView pv = partial_view<D, G>(a.ml + pbase * 2, a.acc + pbase * D, a.max_split);
    publish_partial<D, G>(pv, a.max_split, split, &red.acc[0][0][0], red.M, red.L);
    __syncthreads();
    __shared__ int is_last;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(a.counters + hb, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      is_last = prev == (uint32_t)(a.n_split - 1);
    }
    __syncthreads();
    if (!is_last) return;
    __shared__ MergeLds<64 * NW> mlds;
    merge_splits<D, G, 64 * NW>(mlds, pv, a.max_split, a.n_split,
                                a.out + ((int64_t)b * a.Hq + kvh * G) * D);
    if (threadIdx.x == 0)
      __hip_atomic_store(a.counters + hb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // streaming head: ring slots after the append hold exactly the keys the
    // Lambda mask allows for the new token
    const int hs = kvh - a.Hr;
    const int W = a.S + a.R;
    const int nslots = n + 1 < W ? n + 1 : W;
    const int slot_new = n < a.S ? n : a.S + (n - a.S) % a.R;
    const int64_t hb = (int64_t)b * a.Hs + hs;
    const uint16_t* kr = a.kr + hb * W * D;
    const uint16_t* vr = a.vr + hb * W * D;
    auto kp = [=](int row) { return row == slot_new ? knew : kr + (int64_t)row * D; };
    auto vp = [=](int row) { return row == slot_new ? vnew : vr + (int64_t)row * D; };
    attend_rows<D, G, Tag, NW>(st, qf, 0, nslots, kp, vp);
    if (threadIdx.x < LPR) {
      st16(a.kr + (hb * W + slot_new) * D + threadIdx.x * 8, ld16(knew + threadIdx.x * 8));
      st16(a.vr + (hb * W + slot_new) * D + threadIdx.x * 8, ld16(vnew + threadIdx.x * 8));
    }
    block_merge<D, G, NW>(red, st);
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      int g = i / D, dd = i % D;
      a.out[((int64_t)b * a.Hq + kvh * G + g) * D + dd] =
          (uint16_t)f2bf(red.acc[0][g][dd] / red.L[g]);
    }
  }
}

template <int D, int G, typename Tag>
static hipError_t launch_t(DecodeArgs a, int B, int64_t rows, int split_tokens, int max_split,
                           hipStream_t s) {
  a.split_tokens = split_tokens;
  a.n_split = a.Hr > 0 ? (int)((rows + split_tokens - 1) / split_tokens) : 0;
  if (a.n_split > max_split) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.Hr * a.n_split + a.Hs), (unsigned)B);
  decode_kernel<D, G, Tag><<<grid, 64 * kDecodeWaves, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, typename Tag>
static hipError_t launch_g(int G, const DecodeArgs& a, int B, int64_t rows, int st,
                           int max_split, hipStream_t s) {
  switch (G) {
    case 1: return launch_t<D, 1, Tag>(a, B, rows, st, max_split, s);
    case 2: return launch_t<D, 2, Tag>(a, B, rows, st, max_split, s);
    case 4: return launch_t<D, 4, Tag>(a, B, rows, st, max_split, s);
    default: return launch_t<D, 8, Tag>(a, B, rows, st, max_split, s);
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
  a.ragged = L->ragged ? 1 : 0;
  // ragged positions travel in the arguments: larger batches come in slices
  if (L->ragged && d.batch > kMaxRaggedBatch) return hipErrorInvalidValue;
  for (int b = 0; b < d.batch && b < kMaxRaggedBatch; ++b) a.nseq[b] = (int)L->nseq[b];
  a.qscale = d.softmax_scale * kLog2e;
  const int64_t rows = L->n + 1;  // the longest sequence
  const int B = d.batch;
  const int st = decode_split_tokens(L, rows, 1, L->cus * 4 / 5);
  const int ms = L->max_split;
  if (d.head_dim == 128) {
    if (d.kv_dtype == DUO_FP16) return launch_g<128, Fp16Tag>(L->G, a, B, rows, st, ms, s);
    return launch_g<128, Bf16Tag>(L->G, a, B, rows, st, ms, s);
  }
  if (d.kv_dtype == DUO_FP16) return launch_g<64, Fp16Tag>(L->G, a, B, rows, st, ms, s);
  return launch_g<64, Bf16Tag>(L->G, a, B, rows, st, ms, s);
}

}  // namespace duo

