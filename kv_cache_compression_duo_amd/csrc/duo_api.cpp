// C-ABI front end: argument validation, buffer layout, host token counter and
// dispatch to the kernel launchers. Every check runs before any HIP call, so
// a failed call enqueues nothing and leaves the layer unchanged.
#include <math.h>
#include <algorithm>
#include <initializer_list>
#include <new>
#include <vector>
#include <stdlib.h>
#include <string.h>

#include "duo_internal.hpp"

namespace duo {

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int max_split_for(const duo_layer_desc& d) {
  int64_t cap = d.retrieval_capacity;
  int64_t s = (cap + kMinSplitTokens - 1) / kMinSplitTokens + 1;
  return (int)(s < 1 ? 1 : s);
}

// Split count: the launch gets at most `blocks` blocks, `blocks` no more
// than the compute units (a CU that gets two long blocks while others get
// one sets the step time: 8 blocks more than CUs made a plain read 40 %
// slower, and 32 splits per head of the Llama-2 layer, 280 blocks, 33 %).
// The memory-bound 16-bit decode asks for 4/5 of the CUs (measured on the
// Llama-2 layer: 24 splits per head, 216 blocks, 2.5 % faster than 31); the
// VALU-bound 4-bit decode asks for all of them (63 splits per head 10 %
// faster than 48). Streaming-head blocks read at most S + R rows, so four of
// them are counted as one block. DUO_DECODE_SPLIT_TOKENS, if set to a
// positive value, overrides the rule.
static int split_tokens_override() {
  const char* e = getenv("DUO_DECODE_SPLIT_TOKENS");
  const int v = e ? atoi(e) : 0;
  return v > 0 ? v : 0;
}

int decode_split_tokens(const duo_layer* L, int64_t rows, int tile, int blocks) {
  // read once; the initialisation of a local static is thread-safe
  static const int env = split_tokens_override();
  int64_t st = env;
  if (st <= 0) {
    const int B = L->d.batch;
    int64_t per_head = (int64_t)(blocks - (B * L->Hs) / 4) / ((int64_t)B * (L->Hr > 0 ? L->Hr : 1));
    if (per_head < 1) per_head = 1;
    st = (rows + per_head - 1) / per_head;
  }
  st = (st + tile - 1) / tile * tile;
  if (st < kMinSplitTokens) st = kMinSplitTokens;
  if (st > (int64_t)1 << 30) st = (int64_t)1 << 30;
  return (int)st;
}

size_t ws_bytes(const duo_layer_desc& d, int max_split) {
  size_t Hr = (size_t)d.n_retrieval_kv_heads, B = (size_t)d.batch;
  size_t G = (size_t)(d.n_q_heads / d.n_kv_heads);
  size_t cnt = align_up(B * Hr * sizeof(uint32_t) + 4, 256);
  size_t ml = align_up(B * Hr * G * (size_t)max_split * 2 * sizeof(float), 256);
  size_t acc = align_up(B * Hr * G * (size_t)max_split * (size_t)d.head_dim * sizeof(float), 256);
  return cnt + ml + acc;
}

WsView ws_view(const duo_layer* L) {
  // the attached layer's batch, not a view's: every view of a layer must
  // find the counters and partials at the same offsets
  size_t Hr = (size_t)L->Hr, B = (size_t)L->ws_batch, G = (size_t)L->G;
  size_t cnt = align_up(B * Hr * sizeof(uint32_t) + 4, 256);
  size_t ml = align_up(B * Hr * G * (size_t)L->max_split * 2 * sizeof(float), 256);
  WsView v;
  v.counters = reinterpret_cast<uint32_t*>(L->ws);
  v.ml = reinterpret_cast<float*>(L->ws + cnt);
  v.acc = reinterpret_cast<float*>(L->ws + cnt + ml);
  return v;
}

// Heads per block of the flash kernels for group size G (as their launcher
// picks: 1 for G = 1, 2 for G = 2, 4 for G = 4 or 8).
int heads_per_block(int G) { return G == 1 ? 1 : (G == 2 ? 2 : 4); }

// One partial sum per flash block of the gate gradient: 8 waves of 32 query
// rows per block, heads_per_block heads sharing a block.
size_t mixed_grad_partials(const duo_layer_desc& d, int T) {
  const int G = d.n_q_heads / d.n_kv_heads, HB = heads_per_block(G);
  const int BMT = 32 * 8 / HB;
  return (size_t)d.batch * d.n_kv_heads * (G / HB) * (size_t)((T + BMT - 1) / BMT);
}

// true when the product of the factors stays at or below 2^62 bytes (no
// buffer of a layer is larger; the bound also keeps every sum of such
// products below 2^64)
static bool size_ok(std::initializer_list<size_t> factors) {
  size_t r = 1;
  for (size_t x : factors)
    if (__builtin_mul_overflow(r, x, &r) || r > ((size_t)1 << 62)) return false;
  return true;
}

static duo_status check_desc(const duo_layer_desc* d) {
  if (!d) return DUO_ERR_INVALID_ARG;
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return DUO_ERR_INVALID_ARG;
  // the batch index and a cache's head index are grid dimensions of at most
  // 65535 blocks (checked here so that no launch of a call can fail on them
  // after an earlier launch of the same call was enqueued)
  if (d->batch > 65535 || d->n_kv_heads > 65535) return DUO_ERR_UNSUPPORTED;
  if (d->n_q_heads % d->n_kv_heads) return DUO_ERR_INVALID_ARG;
  int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return DUO_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return DUO_ERR_UNSUPPORTED;
  if (d->n_retrieval_kv_heads < 0 || d->n_retrieval_kv_heads > d->n_kv_heads)
    return DUO_ERR_INVALID_ARG;
  if (d->sink < 0 || d->recent < 1) return DUO_ERR_INVALID_ARG;
  if ((int64_t)d->sink + d->recent > 1024) return DUO_ERR_UNSUPPORTED;
  if (d->retrieval_capacity < 0 || d->retrieval_capacity > (int64_t)INT32_MAX)
    return DUO_ERR_INVALID_ARG;
  if (d->kv_dtype != DUO_BF16 && d->kv_dtype != DUO_FP16) return DUO_ERR_UNSUPPORTED;
  if (d->retrieval_dtype != d->kv_dtype && d->retrieval_dtype != DUO_INT4_G32)
    return DUO_ERR_UNSUPPORTED;
  if (!isfinite(d->softmax_scale) || !(d->softmax_scale > 0.0f)) return DUO_ERR_INVALID_ARG;
  // every buffer size of the layout must be representable
  {
    const size_t B = (size_t)d->batch, D = (size_t)d->head_dim;
    const size_t cap = (size_t)cap32_of(d->retrieval_capacity) + kDecodePadRows;
    const size_t G = (size_t)(d->n_q_heads / d->n_kv_heads);
    if (!size_ok({B, (size_t)d->n_kv_heads, cap, D, 4}) ||
        !size_ok({B, (size_t)d->n_kv_heads, (size_t)(d->sink + d->recent), D, 4}) ||
        !size_ok({B, (size_t)d->n_kv_heads, G, (size_t)max_split_for(*d), D + 2, 4}))
      return DUO_ERR_CAPACITY;
  }
  // the split-K partials of one (sequence, KV head) are addressed with 32-bit
  // byte offsets (implied by the cache limits below; checked here as well)
  if ((int64_t)G * max_split_for(*d) * (d->head_dim + 2) * 4 >= ((int64_t)1 << 31))
    return DUO_ERR_UNSUPPORTED;
  // the 4-bit decode kernel maps (query head, channel group) pairs of a KV
  // head onto the 16 columns of one MFMA tile
  if (d->retrieval_dtype == DUO_INT4_G32 && G * (d->head_dim / 32) > 16) return DUO_ERR_UNSUPPORTED;
  // ... and addresses one head's code array with 32-bit offsets
  if (d->retrieval_dtype == DUO_INT4_G32 &&
      cap32_of(d->retrieval_capacity) * (d->head_dim / 2) >= ((int64_t)1 << 31))
    return DUO_ERR_UNSUPPORTED;
  // the 16-bit decode kernel reads one head's rows (plus the padding rows)
  // as one buffer resource with 32-bit byte offsets
  if (d->retrieval_dtype != DUO_INT4_G32 &&
      (d->retrieval_capacity + kDecodePadRows) * d->head_dim * 2 >= ((int64_t)1 << 31))
    return DUO_ERR_UNSUPPORTED;
  return DUO_OK;
}

}  // namespace duo

using namespace duo;

extern "C" {

duo_status duo_layer_layout(const duo_layer_desc* d, duo_layout* out) {
  duo_status st = check_desc(d);
  if (st != DUO_OK) return st;
  if (!out) return DUO_ERR_INVALID_ARG;
  size_t B = (size_t)d->batch, D = (size_t)d->head_dim, cap = (size_t)d->retrieval_capacity;
  size_t Hr = (size_t)d->n_retrieval_kv_heads, Hs = (size_t)(d->n_kv_heads - d->n_retrieval_kv_heads);
  size_t W = (size_t)(d->sink + d->recent);
  duo_layout L;
  memset(&L, 0, sizeof(L));
  if (d->retrieval_dtype == DUO_INT4_G32) {
    const size_t cap32 = (size_t)cap32_of(d->retrieval_capacity);
    size_t codes = align_up(B * Hr * cap32 * (D / 2), 256);
    size_t sz = align_up(B * Hr * cap32 * (D / 32) * 2 * 2, 256);
    L.k_offset = 0;
    L.v_offset = codes;
    L.k_sz_offset = 2 * codes;
    L.v_sz_offset = 2 * codes + sz;
    L.retrieval_bytes = 2 * codes + 2 * sz;
  } else {
    size_t arr = align_up(B * Hr * cap * D * 2, 256);
    L.k_offset = 0;
    L.v_offset = arr;
    L.k_sz_offset = L.v_sz_offset = 0;
    // the decode kernel reads whole row tiles from any valid start row, so
    // the buffer extends kDecodePadRows rows past the last V row
    L.retrieval_bytes = Hr ? 2 * arr + align_up((size_t)kDecodePadRows * D * 2, 256) : 0;
  }
  size_t ring = align_up(B * Hs * W * D * 2, 256);
  L.ring_k_offset = 0;
  L.ring_v_offset = ring;
  L.streaming_bytes = 2 * ring;
  L.workspace_bytes = ws_bytes(*d, max_split_for(*d));
  *out = L;
  return DUO_OK;
}

static duo_status layer_init(duo_layer** out, const duo_layer_desc* d, void* retrieval_buf,
                             void* streaming_buf, void* workspace, const int64_t* n_existing,
                             int64_t n_uniform, hipStream_t stream) {
  if (!out) return DUO_ERR_INVALID_ARG;
  duo_layout lay;
  duo_status st = duo_layer_layout(d, &lay);
  if (st != DUO_OK) return st;
  int64_t n_max = 0;
  bool ragged = false;
  for (int32_t b = 0; b < d->batch; ++b) {
    const int64_t nb = n_existing ? n_existing[b] : n_uniform;
    if (nb < 0) return DUO_ERR_INVALID_ARG;
    if (d->n_retrieval_kv_heads > 0 && nb > d->retrieval_capacity) return DUO_ERR_CAPACITY;
    if (nb > (int64_t)INT32_MAX) return DUO_ERR_CAPACITY;
    if (b > 0 && nb != n_max) ragged = true;
    if (b == 0 || nb > n_max) n_max = nb;
  }
  if (lay.retrieval_bytes && !retrieval_buf) return DUO_ERR_INVALID_ARG;
  if (lay.streaming_bytes && !streaming_buf) return DUO_ERR_INVALID_ARG;
  if (!workspace) return DUO_ERR_INVALID_ARG;
  if (!aligned(retrieval_buf, 256) || !aligned(streaming_buf, 256) || !aligned(workspace, 256))
    return DUO_ERR_LAYOUT;
  duo_layer* L = new (std::nothrow) duo_layer;
  if (!L) return DUO_ERR_INVALID_ARG;
  L->nseq = new (std::nothrow) int64_t[(size_t)d->batch];
  if (!L->nseq) {
    delete L;
    return DUO_ERR_INVALID_ARG;
  }
  for (int32_t b = 0; b < d->batch; ++b) L->nseq[b] = n_existing ? n_existing[b] : n_uniform;
  L->n = n_max;
  L->ragged = ragged;
  L->d = *d;
  L->lay = lay;
  L->rbuf = static_cast<char*>(retrieval_buf);
  L->sbuf = static_cast<char*>(streaming_buf);
  L->ws = static_cast<char*>(workspace);
  L->G = d->n_q_heads / d->n_kv_heads;
  L->Hr = d->n_retrieval_kv_heads;
  L->Hs = d->n_kv_heads - d->n_retrieval_kv_heads;
  L->max_split = max_split_for(*d);
  L->ws_batch = d->batch;
  int dev = 0;
  L->cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&L->cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      L->cus <= 0)
    L->cus = 256;
  if (launch_zero(workspace, lay.workspace_bytes, stream) != hipSuccess) {
    delete[] L->nseq;
    delete L;
    return DUO_ERR_HIP;
  }
  *out = L;
  return DUO_OK;
}

duo_status duo_layer_init(duo_layer** out, const duo_layer_desc* d, void* retrieval_buf,
                          void* streaming_buf, void* workspace, int64_t n_tokens_existing,
                          hipStream_t stream) {
  return layer_init(out, d, retrieval_buf, streaming_buf, workspace, nullptr, n_tokens_existing,
                    stream);
}

duo_status duo_layer_init_ragged(duo_layer** out, const duo_layer_desc* d, void* retrieval_buf,
                                 void* streaming_buf, void* workspace,
                                 const int64_t* n_tokens_existing, hipStream_t stream) {
  if (!n_tokens_existing) return DUO_ERR_INVALID_ARG;
  return layer_init(out, d, retrieval_buf, streaming_buf, workspace, n_tokens_existing, 0,
                    stream);
}

duo_status duo_layer_destroy(duo_layer* L) {
  if (L) delete[] L->nseq;
  delete L;
  return DUO_OK;
}

int64_t duo_layer_tokens(const duo_layer* L) { return L ? L->n : -1; }

int64_t duo_layer_sequence_tokens(const duo_layer* L, int32_t b) {
  if (!L || b < 0 || b >= L->d.batch) return -1;
  return L->nseq[b];
}

static duo_status check_act(const void* p) {
  if (!p) return DUO_ERR_INVALID_ARG;
  if (!aligned(p, 16)) return DUO_ERR_LAYOUT;
  return DUO_OK;
}

// Every sequence grew by T tokens.
static void advance_all(duo_layer* L, int64_t T) {
  for (int32_t b = 0; b < L->d.batch; ++b) L->nseq[b] += T;
  L->n += T;
}

static duo_status prefill_launch(duo_layer* L, const void* q, const void* k, const void* v,
                                 int32_t T, void* out, hipStream_t stream);

duo_status duo_append_kv(duo_layer* L, const void* k, const void* v, int32_t T,
                         hipStream_t stream) {
  if (!L || T < 1) return DUO_ERR_INVALID_ARG;
  duo_status st;
  if ((st = check_act(k)) != DUO_OK || (st = check_act(v)) != DUO_OK) return st;
  if (L->ragged) return DUO_ERR_UNSUPPORTED;  // per sequence: duo_append_kv_seq
  if (L->Hr > 0 && L->n + T > L->d.retrieval_capacity) return DUO_ERR_CAPACITY;
  if (L->n + T > (int64_t)INT32_MAX) return DUO_ERR_CAPACITY;
  if (L->Hr > 0 && launch_append_cache(L, k, v, T, stream) != hipSuccess) return DUO_ERR_HIP;
  if (L->Hs > 0 && launch_append_ring(L, k, v, T, stream) != hipSuccess) return DUO_ERR_HIP;
  advance_all(L, T);
  return DUO_OK;
}

duo_status duo_prefill_chunk(duo_layer* L, const void* q, const void* k, const void* v,
                             int32_t T, void* out, hipStream_t stream) {
  if (!L || T < 1) return DUO_ERR_INVALID_ARG;
  duo_status st;
  if ((st = check_act(q)) != DUO_OK || (st = check_act(k)) != DUO_OK ||
      (st = check_act(v)) != DUO_OK || (st = check_act(out)) != DUO_OK)
    return st;
  if (L->ragged) return DUO_ERR_UNSUPPORTED;  // per sequence: duo_prefill_chunk_seq
  if (L->Hr > 0 && L->n + T > L->d.retrieval_capacity) return DUO_ERR_CAPACITY;
  if (L->n + T > (int64_t)INT32_MAX) return DUO_ERR_CAPACITY;
  if ((st = prefill_launch(L, q, k, v, T, out, stream)) != DUO_OK) return st;
  advance_all(L, T);
  return DUO_OK;
}

// The batch-wide prefill of a (view of a) layer, after validation; leaves the
// token counts to the caller (a view shares its parent's count array).
static duo_status prefill_launch(duo_layer* L, const void* q, const void* k, const void* v,
                                 int32_t T, void* out, hipStream_t stream) {
  // Retrieval heads: append the chunk, then attend causally over the cache.
  if (L->Hr > 0) {
    if (launch_append_cache(L, k, v, T, stream) != hipSuccess) return DUO_ERR_HIP;
    if (launch_prefill_retrieval(L, q, T, out, stream) != hipSuccess) return DUO_ERR_HIP;
  }
  // Streaming heads: attend over the ring as it was before the chunk plus the
  // chunk, then update the ring (the chunk overwrites slots still being read).
  if (L->Hs > 0) {
    if (launch_prefill_streaming(L, q, k, v, T, out, stream) != hipSuccess) return DUO_ERR_HIP;
    if (launch_append_ring(L, k, v, T, stream) != hipSuccess) return DUO_ERR_HIP;
  }
  return DUO_OK;  // the caller advances the token counts
}

static duo_layer batch_view(const duo_layer* L, int32_t b0, int32_t nb);

duo_status duo_decode(duo_layer* L, const void* q, const void* k_new, const void* v_new,
                      void* out, hipStream_t stream) {
  if (!L) return DUO_ERR_INVALID_ARG;
  duo_status st;
  if ((st = check_act(q)) != DUO_OK || (st = check_act(k_new)) != DUO_OK ||
      (st = check_act(v_new)) != DUO_OK || (st = check_act(out)) != DUO_OK)
    return st;
  if (L->Hr > 0 && L->n + 1 > L->d.retrieval_capacity) return DUO_ERR_CAPACITY;
  if (L->n + 1 > (int64_t)INT32_MAX) return DUO_ERR_CAPACITY;
  auto launch = [&](const duo_layer* V, size_t b0) {
    const size_t qrow = (size_t)V->d.n_q_heads * V->d.head_dim * 2;
    const size_t kvrow = (size_t)V->d.n_kv_heads * V->d.head_dim * 2;
    const char* qb = static_cast<const char*>(q) + b0 * qrow;
    const char* kb = static_cast<const char*>(k_new) + b0 * kvrow;
    const char* vb = static_cast<const char*>(v_new) + b0 * kvrow;
    char* ob = static_cast<char*>(out) + b0 * qrow;
    return V->d.retrieval_dtype == DUO_INT4_G32 && V->Hr > 0
               ? launch_decode_int4(V, qb, kb, vb, ob, stream)
               : launch_decode(V, qb, kb, vb, ob, stream);
  };
  hipError_t e = hipSuccess;
  if (L->ragged && L->d.batch > kMaxRaggedBatch) {
    // the kernels take ragged positions in their arguments: decode the batch
    // in slices of at most kMaxRaggedBatch sequences, one launch each
    for (int32_t b0 = 0; b0 < L->d.batch && e == hipSuccess; b0 += kMaxRaggedBatch) {
      const duo_layer view = batch_view(L, b0, std::min(kMaxRaggedBatch, L->d.batch - b0));
      e = launch(&view, (size_t)b0);
    }
  } else {
    e = launch(L, 0);
  }
  if (e != hipSuccess) return DUO_ERR_HIP;
  advance_all(L, 1);
  return DUO_OK;
}

// A view of sequences [b0, b0 + nb) of a layer: the same buffers at those
// sequences' offsets (every array is laid out batch-major), their counts,
// and the workspace from its start (calls on one layer are ordered on the
// stream and every decode launch leaves its arrival counters at zero, so
// consecutive launches of views may share it).
static duo_layer batch_view(const duo_layer* L, int32_t b0, int32_t nb) {
  duo_layer v = *L;
  const duo_layer_desc& d = L->d;
  const size_t D = (size_t)d.head_dim, Hr = (size_t)L->Hr, Hs = (size_t)L->Hs;
  const size_t W = (size_t)(d.sink + d.recent), bb = (size_t)b0;
  if (d.retrieval_dtype == DUO_INT4_G32) {
    const size_t cap32 = (size_t)cap32_of(d.retrieval_capacity);
    const size_t codes = Hr * cap32 * (D / 2), sz = Hr * cap32 * (D / 32) * 4;
    v.lay.k_offset += bb * codes;
    v.lay.v_offset += bb * codes;
    v.lay.k_sz_offset += bb * sz;
    v.lay.v_sz_offset += bb * sz;
  } else {
    const size_t arr = Hr * (size_t)d.retrieval_capacity * D * 2;
    v.lay.k_offset += bb * arr;
    v.lay.v_offset += bb * arr;
  }
  const size_t ring = Hs * W * D * 2;
  v.lay.ring_k_offset += bb * ring;
  v.lay.ring_v_offset += bb * ring;
  v.d.batch = nb;
  v.nseq = L->nseq + b0;
  v.n = v.nseq[0];
  v.ragged = false;
  for (int32_t i = 1; i < nb; ++i) {
    if (v.nseq[i] != v.nseq[0]) v.ragged = true;
    if (v.nseq[i] > v.n) v.n = v.nseq[i];
  }
  return v;
}

static duo_layer sequence_view(const duo_layer* L, int32_t b) { return batch_view(L, b, 1); }

// Sequence b grew by T tokens: its count, the maximum, the ragged flag.
static void advance_sequence(duo_layer* L, int32_t b, int64_t T) {
  L->nseq[b] += T;
  int64_t mx = L->nseq[0];
  bool ragged = false;
  for (int32_t i = 1; i < L->d.batch; ++i) {
    if (L->nseq[i] != L->nseq[0]) ragged = true;
    if (L->nseq[i] > mx) mx = L->nseq[i];
  }
  L->n = mx;
  L->ragged = ragged;
}

static duo_status check_sequence(const duo_layer* L, int32_t b, int32_t T) {
  if (!L || b < 0 || b >= L->d.batch || T < 1) return DUO_ERR_INVALID_ARG;
  if (L->Hr > 0 && L->nseq[b] + T > L->d.retrieval_capacity) return DUO_ERR_CAPACITY;
  if (L->nseq[b] + T > (int64_t)INT32_MAX) return DUO_ERR_CAPACITY;
  return DUO_OK;
}

duo_status duo_append_kv_seq(duo_layer* L, int32_t b, const void* k, const void* v, int32_t T,
                             hipStream_t stream) {
  duo_status st = check_sequence(L, b, T);
  if (st != DUO_OK) return st;
  if ((st = check_act(k)) != DUO_OK || (st = check_act(v)) != DUO_OK) return st;
  duo_layer view = sequence_view(L, b);
  if (view.Hr > 0 && launch_append_cache(&view, k, v, T, stream) != hipSuccess)
    return DUO_ERR_HIP;
  if (view.Hs > 0 && launch_append_ring(&view, k, v, T, stream) != hipSuccess)
    return DUO_ERR_HIP;
  advance_sequence(L, b, T);
  return DUO_OK;
}

duo_status duo_prefill_chunk_seq(duo_layer* L, int32_t b, const void* q, const void* k,
                                 const void* v, int32_t T, void* out, hipStream_t stream) {
  duo_status st = check_sequence(L, b, T);
  if (st != DUO_OK) return st;
  if ((st = check_act(q)) != DUO_OK || (st = check_act(k)) != DUO_OK ||
      (st = check_act(v)) != DUO_OK || (st = check_act(out)) != DUO_OK)
    return st;
  duo_layer view = sequence_view(L, b);
  if ((st = prefill_launch(&view, q, k, v, T, out, stream)) != DUO_OK) return st;
  advance_sequence(L, b, T);
  return DUO_OK;
}

duo_status duo_mixed_forward_block(const duo_layer_desc* d, const void* q, const void* k,
                                   const void* v, const float* alpha, int32_t T,
                                   int32_t lambda_block, void* out, hipStream_t stream) {
  duo_status st = check_desc(d);
  if (st != DUO_OK) return st;
  if (d->kv_dtype != DUO_BF16) return DUO_ERR_UNSUPPORTED;
  if (lambda_block != 0 && lambda_block != 64) return DUO_ERR_UNSUPPORTED;
  if (T < 1) return DUO_ERR_INVALID_ARG;
  if ((st = check_act(q)) != DUO_OK || (st = check_act(k)) != DUO_OK ||
      (st = check_act(v)) != DUO_OK || (st = check_act(out)) != DUO_OK)
    return st;
  if (!alpha) return DUO_ERR_INVALID_ARG;
  if (!aligned(alpha, 4)) return DUO_ERR_LAYOUT;
  // the kernel reads one KV head's rows of a sequence through a 32-bit range
  if ((int64_t)T * d->n_kv_heads * d->head_dim * 2 >= ((int64_t)1 << 31))
    return DUO_ERR_UNSUPPORTED;
  if (launch_mixed(*d, q, k, v, alpha, T, lambda_block, out, stream) != hipSuccess)
    return DUO_ERR_HIP;
  return DUO_OK;
}

duo_status duo_mixed_forward(const duo_layer_desc* d, const void* q, const void* k,
                             const void* v, const float* alpha, int32_t T, void* out,
                             hipStream_t stream) {
  return duo_mixed_forward_block(d, q, k, v, alpha, T, 0, out, stream);
}

size_t duo_mixed_alpha_grad_workspace(const duo_layer_desc* d, int32_t T) {
  if (check_desc(d) != DUO_OK || T < 1) return 0;
  return align_up(mixed_grad_partials(*d, T) * sizeof(float), 256);
}

// Checks shared by the gate-gradient calls (everything but the workspace).
static duo_status check_alpha_grad(const duo_layer_desc* d, const void* q, const void* k,
                                   const void* v, const void* dout, const float* alpha,
                                   float l1_weight, int32_t T, int32_t lambda_block,
                                   const float* grad) {
  duo_status st = check_desc(d);
  if (st != DUO_OK) return st;
  if (d->kv_dtype != DUO_BF16) return DUO_ERR_UNSUPPORTED;
  if (lambda_block != 0 && lambda_block != 64) return DUO_ERR_UNSUPPORTED;
  if (T < 1 || !isfinite(l1_weight)) return DUO_ERR_INVALID_ARG;
  if ((st = check_act(q)) != DUO_OK || (st = check_act(k)) != DUO_OK ||
      (st = check_act(v)) != DUO_OK || (st = check_act(dout)) != DUO_OK)
    return st;
  if (!alpha || !grad) return DUO_ERR_INVALID_ARG;
  if (!aligned(alpha, 4) || !aligned(grad, 4)) return DUO_ERR_LAYOUT;
  if ((int64_t)T * d->n_kv_heads * d->head_dim * 2 >= ((int64_t)1 << 31))
    return DUO_ERR_UNSUPPORTED;
  return DUO_OK;
}

duo_status duo_mixed_alpha_grad_block(const duo_layer_desc* d, const void* q, const void* k,
                                      const void* v, const void* dout, const float* alpha,
                                      float l1_weight, int32_t T, int32_t lambda_block,
                                      float* grad, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  duo_status st = check_alpha_grad(d, q, k, v, dout, alpha, l1_weight, T, lambda_block, grad);
  if (st != DUO_OK) return st;
  if (!ws) return DUO_ERR_INVALID_ARG;
  if (!aligned(ws, 16)) return DUO_ERR_LAYOUT;
  if (ws_bytes < mixed_grad_partials(*d, T) * sizeof(float)) return DUO_ERR_INVALID_ARG;
  if (launch_mixed_alpha_grad(*d, q, k, v, dout, alpha, l1_weight, T, lambda_block, grad,
                              static_cast<float*>(ws), stream) != hipSuccess)
    return DUO_ERR_HIP;
  return DUO_OK;
}

duo_status duo_mixed_alpha_grad_noalloc(const duo_layer_desc* d, const void* q, const void* k,
                                        const void* v, const void* dout, const float* alpha,
                                        float l1_weight, int32_t T, int32_t lambda_block,
                                        float* grad, hipStream_t stream) {
  duo_status st = check_alpha_grad(d, q, k, v, dout, alpha, l1_weight, T, lambda_block, grad);
  if (st != DUO_OK) return st;
  if (mixed_grad_partials(*d, T) > kGradScratchPartials) return DUO_ERR_CAPACITY;
  float* partial = nullptr;
  if (grad_scratch(&partial) != hipSuccess) return DUO_ERR_HIP;
  if (launch_mixed_alpha_grad(*d, q, k, v, dout, alpha, l1_weight, T, lambda_block, grad,
                              partial, stream) != hipSuccess)
    return DUO_ERR_HIP;
  return DUO_OK;
}

duo_status duo_mixed_alpha_grad(const duo_layer_desc* d, const void* q, const void* k,
                                const void* v, const void* dout, const float* alpha,
                                float l1_weight, int32_t T, float* grad, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return duo_mixed_alpha_grad_block(d, q, k, v, dout, alpha, l1_weight, T, 0, grad, ws,
                                    ws_bytes, stream);
}

duo_status duo_head_permutation(const uint8_t* mask, int32_t n, int32_t* perm,
                                int32_t* n_retrieval) {
  if (!mask || !perm || !n_retrieval || n < 1) return DUO_ERR_INVALID_ARG;
  int32_t w = 0;
  for (int32_t h = 0; h < n; ++h)
    if (mask[h]) perm[w++] = h;
  *n_retrieval = w;
  for (int32_t h = 0; h < n; ++h)
    if (!mask[h]) perm[w++] = h;
  return DUO_OK;
}

duo_status duo_binarize_gates(const float* alpha, int32_t n, double sparsity, uint8_t* mask) {
  if (!alpha || !mask || n < 1) return DUO_ERR_INVALID_ARG;
  if (!(sparsity >= 0.0 && sparsity <= 1.0)) return DUO_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (isnan(alpha[i])) return DUO_ERR_INVALID_ARG;
  const int64_t n_stream = (int64_t)floor(sparsity * (double)n);
  if (n_stream >= n) {
    memset(mask, 0, (size_t)n);
    return DUO_OK;
  }
  float tau;
  try {  // no exception (an allocation failure) may leave through the C ABI
    std::vector<float> sorted(alpha, alpha + n);
    std::nth_element(sorted.begin(), sorted.begin() + n_stream, sorted.end());
    tau = sorted[(size_t)n_stream];
  } catch (...) {
    return DUO_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) mask[i] = alpha[i] >= tau ? 1 : 0;
  return DUO_OK;
}

duo_status duo_reorder_head_rows(const void* in, void* out, const int32_t* perm, int32_t n_heads,
                                 int64_t rows_per_head, int64_t row_bytes) {
  if (!in || !out || !perm || n_heads < 1 || rows_per_head < 1 || row_bytes < 1)
    return DUO_ERR_INVALID_ARG;
  const size_t block = (size_t)rows_per_head * (size_t)row_bytes;
  const size_t total = block * (size_t)n_heads;
  if (block / (size_t)row_bytes != (size_t)rows_per_head || total / block != (size_t)n_heads)
    return DUO_ERR_INVALID_ARG;
  const char* src = static_cast<const char*>(in);
  char* dst = static_cast<char*>(out);
  if (src < dst + total && dst < src + total) return DUO_ERR_LAYOUT;  // overlapping buffers
  try {  // as above: allocation failures become a status
    std::vector<uint8_t> seen((size_t)n_heads, 0);
    for (int32_t i = 0; i < n_heads; ++i) {
      if (perm[i] < 0 || perm[i] >= n_heads || seen[(size_t)perm[i]]) return DUO_ERR_INVALID_ARG;
      seen[(size_t)perm[i]] = 1;
    }
  } catch (...) {
    return DUO_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n_heads; ++i)
    memcpy(dst + (size_t)i * block, src + (size_t)perm[i] * block, block);
  return DUO_OK;
}

int32_t duo_ring_slot(int64_t p, int32_t sink, int32_t recent) {
  if (p < 0 || sink < 0 || recent < 1) return -1;
  if (p < sink) return (int32_t)p;
  return (int32_t)(sink + (p - sink) % recent);
}

const char* duo_status_string(duo_status s) {
  switch (s) {
    case DUO_OK: return "ok";
    case DUO_ERR_INVALID_ARG: return "invalid argument";
    case DUO_ERR_UNSUPPORTED: return "unsupported configuration";
    case DUO_ERR_LAYOUT: return "bad layout or alignment";
    case DUO_ERR_CAPACITY: return "retrieval cache capacity exceeded";
    case DUO_ERR_HIP: return "HIP launch or API error";
  }
  return "unknown status";
}

}  // extern "C"
