// Internal declarations shared by the C-ABI front end and the kernel launchers.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/duo.h"

struct duo_layer {
  duo_layer_desc d;
  duo_layout lay;
  char* rbuf;
  char* sbuf;
  char* ws;
  int64_t n;      // tokens cached: the largest count over the batch's sequences
  int64_t* nseq;  // tokens cached per sequence [batch] (owned)
  bool ragged;    // the sequences' counts differ
  int G, Hr, Hs;  // group size, retrieval / streaming KV heads
  int max_split;  // split-K partial slots per retrieval (batch, KV head)
  int ws_batch;   // batch the workspace is laid out for: the attached layer's,
                  // kept by views of some of its sequences
  int cus;        // compute units of the device the layer was attached on
};

namespace duo {

// Workspace layout: [counters: B*Hr u32, padded to 256 B][m,l: B*Hr*G*max_split*2 f32]
//                   [acc: B*Hr*G*max_split*D f32], B the batch of the layer the
// workspace was attached with (a view of fewer sequences keeps that layout and
// uses the leading entries of each region).
constexpr int kMinSplitTokens = 256;  // smallest split-K range (tokens)
// Layers whose sequences hold different token counts pass the counts to the
// decode kernels in their arguments: at most this many sequences.
constexpr int kMaxRaggedBatch = 64;
// Rows of readable (never used) memory after a bf16/fp16 retrieval buffer: a
// decode tile (at most 32 rows) starting at any valid row stays inside the buffer.
constexpr int kDecodePadRows = 32;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
// 4-bit caches are allocated in whole 32-token blocks.
inline int64_t cap32_of(int64_t cap) { return (cap + 31) / 32 * 32; }

struct WsView {
  uint32_t* counters;
  float* ml;
  float* acc;
};
WsView ws_view(const duo_layer* L);
size_t ws_bytes(const duo_layer_desc& d, int max_split);
int max_split_for(const duo_layer_desc& d);
// Split-K range (tokens, a multiple of `tile`, at least kMinSplitTokens) of a
// decode step over `rows` cache rows.
int decode_split_tokens(const duo_layer* L, int64_t rows, int tile, int blocks);

// ---- launchers (return hipSuccess or the launch error) ----------------------
hipError_t launch_append_cache(const duo_layer* L, const void* k, const void* v, int T,
                               hipStream_t s);
hipError_t launch_append_ring(const duo_layer* L, const void* k, const void* v, int T,
                              hipStream_t s);
hipError_t launch_decode(const duo_layer* L, const void* q, const void* k_new,
                         const void* v_new, void* out, hipStream_t s);
hipError_t launch_decode_int4(const duo_layer* L, const void* q, const void* k_new,
                              const void* v_new, void* out, hipStream_t s);
hipError_t launch_prefill_retrieval(const duo_layer* L, const void* q, int T, void* out,
                                    hipStream_t s);
hipError_t launch_prefill_streaming(const duo_layer* L, const void* q, const void* k,
                                    const void* v, int T, void* out, hipStream_t s);
hipError_t launch_mixed(const duo_layer_desc& d, const void* q, const void* k, const void* v,
                        const float* alpha, int T, int lam_block, void* out, hipStream_t s);
// gate gradient of the gate-blended forward: partial sums per flash block
// (mixed_grad_partials floats), then one reduction launch
int heads_per_block(int G);
size_t mixed_grad_partials(const duo_layer_desc& d, int T);
hipError_t launch_mixed_alpha_grad(const duo_layer_desc& d, const void* q, const void* k,
                                   const void* v, const void* dout, const float* alpha,
                                   float l1_weight, int T, int lam_block, float* grad,
                                   float* partial, hipStream_t s);
// Partial slots of the allocation-free gate gradient (a file-scope device
// array; duo_mixed_alpha_grad_noalloc refuses larger launches).
constexpr size_t kGradScratchPartials = DUO_GRAD_SCRATCH_PARTIALS;
// Address of the current device's copy of that array (looked up on first use).
hipError_t grad_scratch(float** out);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace duo
